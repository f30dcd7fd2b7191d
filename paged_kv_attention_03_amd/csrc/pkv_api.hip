// C ABI of the paged-KV attention library (declared in include/pkv.h).
//
// Host side: argument validation (before any launch), the launch planner
// (which sequences take the decode or the prefill path, the split size of the
// decode pass, workspace layout), kernel launches on the caller's stream, and
// host-copy metadata checkers.  The library allocates nothing and never
// synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "pkv.h"
#include "append.hpp"
#include "decode.hpp"
#include "prefill.hpp"
#include "step.hpp"
#include "cascade.hpp"
#include "pool.hpp"

struct pkv_pool {
    pkv::PagePool pool;
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return PKV_OK;
}

int hip_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return PKV_OK;
}

size_t elem_bytes(pkv_dtype_t dt) { return dt == PKV_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return na && nb && x < y + nb && y < x + na;
}

// ---------------------------------------------------------------- planner

// Workspace layout (every region 256-byte aligned):
//   pair_prefix   int32[num_seqs + 1]          page pairs of decode sequences before s
//   portion_begin int32[kDecodeWaves + 1]      each wave's first segment piece
//   portions      Portion[kDecodeWaves + num_seqs * Hkv]
//   ws_o          float[kDecodeWaves * 2][ncol][D] partial outputs of cut segments
//   ws_ml         float[kDecodeWaves * 2][ncol][2] their running max and sum
// ncol = G * wmax: the query rows of one kv head in a sequence of the decode
// path (up to wmax = min(16 / G, max_seqlen_q) query tokens).
struct Plan {
    size_t off_prefix = 0, off_pbegin = 0, off_portions = 0, off_o = 0, off_ml = 0, total = 0;
    int prefill_tile_tokens = 0;
    int wmax = 1;  // sequences with 1..wmax query tokens take the decode path
};

constexpr int kBlock = 16;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Query tokens a sequence of the decode path may have: its G * n query rows
// must fit the 16 columns of one matrix-core tile.
int decode_window(int group, int max_seqlen_q) {
    return std::max(1, std::min(16 / group, max_seqlen_q));
}

Plan make_plan(int num_seqs, int num_kv_heads, int head_dim, int group, int max_seqlen_q) {
    Plan pl;
    pl.wmax = decode_window(group, max_seqlen_q);
    const size_t ncol = (size_t)group * pl.wmax;
    size_t off = 0;
    pl.off_prefix = off;
    off = align256(off + sizeof(int32_t) * (size_t)(num_seqs + 1));
    pl.off_pbegin = off;
    off = align256(off + sizeof(int32_t) * (size_t)(pkv::kDecodeWaves + 1));
    pl.off_portions = off;
    off = align256(off + sizeof(pkv::Portion) * ((size_t)pkv::kDecodeWaves + (size_t)num_seqs * num_kv_heads));
    pl.off_o = off;
    off = align256(off + sizeof(float) * (size_t)pkv::kDecodeWaves * 2 * ncol * head_dim);
    pl.off_ml = off;
    off = align256(off + sizeof(float) * (size_t)pkv::kDecodeWaves * 2 * ncol * 2);
    pl.total = off;
    pl.prefill_tile_tokens = pkv::kPrefillRows / group;
    return pl;
}

// Shared-prefix steps: the workspace after the plain plan holds the setup
// kernel's outputs and the prefix states (every region 256-byte aligned):
//   kv_eff int32[num_seqs], prefix_states int4[num_seqs],
//   v_qsl int32[V + 1], v_lens, v_start, v_row int32[V], v_qrows int32[V * M],
//   state float[V * M][Hq][D + 4],
// V = groups x chunks per group, M = max_group_size.  Chunks are sized so
// that the prefix pass has about one workgroup per CU: groups x chunks x kv
// heads ~ 256, at least 64 keys, a multiple of 32 (whole page pairs).
struct CascadePlan {
    int chunk = 0, max_chunks = 0, V = 0;
    int64_t vtokens = 0;
    size_t off_kv = 0, off_states = 0, off_vqsl = 0, off_vlens = 0, off_vstart = 0, off_vrow = 0,
           off_vqrows = 0, off_state = 0, total = 0;
};

CascadePlan make_cascade_plan(size_t base, int num_seqs, int num_groups, int max_group_size,
                              int max_prefix_len, int num_q_heads, int num_kv_heads, int head_dim) {
    CascadePlan c;
    const int64_t want = ((int64_t)max_prefix_len * num_groups * num_kv_heads + 255) / 256;
    c.chunk = (int)std::max<int64_t>(64, (want + 31) / 32 * 32);
    c.max_chunks = (max_prefix_len + c.chunk - 1) / c.chunk;
    c.V = num_groups * c.max_chunks;
    c.vtokens = (int64_t)c.V * max_group_size;
    size_t off = align256(base);
    c.off_kv = off;
    off = align256(off + sizeof(int32_t) * (size_t)num_seqs);
    c.off_states = off;
    off = align256(off + sizeof(int4) * (size_t)num_seqs);
    c.off_vqsl = off;
    off = align256(off + sizeof(int32_t) * (size_t)(c.V + 1));
    c.off_vlens = off;
    off = align256(off + sizeof(int32_t) * (size_t)c.V);
    c.off_vstart = off;
    off = align256(off + sizeof(int32_t) * (size_t)c.V);
    c.off_vrow = off;
    off = align256(off + sizeof(int32_t) * (size_t)c.V);
    c.off_vqrows = off;
    off = align256(off + sizeof(int32_t) * (size_t)c.vtokens);
    c.off_state = off;
    off = align256(off + sizeof(float) * (size_t)c.vtokens * num_q_heads *
                             (size_t)(head_dim + 4));
    c.total = off;
    return c;
}

int check_common(int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                 pkv_dtype_t dtype) {
    if (dtype != PKV_F32 && dtype != PKV_BF16)
        return fail(PKV_E_UNSUPPORTED, "dtype %d is not supported (PKV_F32 or PKV_BF16)", (int)dtype);
    if (num_q_heads <= 0 || num_kv_heads <= 0)
        return fail(PKV_E_ARG, "head counts must be positive (q %d, kv %d)", num_q_heads, num_kv_heads);
    if (num_q_heads % num_kv_heads != 0)
        return fail(PKV_E_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                    num_kv_heads);
    if (num_q_heads / num_kv_heads > 16)
        return fail(PKV_E_UNSUPPORTED, "group size %d > 16 is not supported",
                    num_q_heads / num_kv_heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(PKV_E_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", head_dim);
    if (block_size != kBlock)
        return fail(PKV_E_UNSUPPORTED, "block_size %d is not supported (16)", block_size);
    return PKV_OK;
}

// One tile per (sequence, kv head, 128/G query tokens); the grid is sized from
// host bounds and tiles past a sequence's tokens return at once.
long prefill_tiles(const pkv::PrefillParams& pp) {
    return pp.state ? (long)pp.num_seqs * pp.sp_tiles
                    : (pp.total_q + pp.tile_tokens - 1) / pp.tile_tokens + pp.num_seqs;
}

// A tile's pages: at most ceil(max_seqlen_k / 16) + 1, rounded up to pairs,
// beyond the LDS id table (or a pool whose (page, kv head) offsets / 256
// exceed 32 bits): the variant that reads block ids through the scalar cache.
template <typename T, int D>
bool prefill_long(const pkv::PrefillParams& pp) {
    return ((long)pp.max_seqlen_k + kBlock - 1) / kBlock + 2 > pkv::kPrefillIdTable ||
           (uint64_t)pp.num_blocks * (uint64_t)pp.Hkv * (pkv::PrefillGeom<T, D>::PAGE / 256) >
               0xffffffffull;
}

// Whether a step with prefill sequences runs as one launch (step_kernel:
// decode waves and prefill tiles in one grid) or as separate decode and
// prefill launches.  One launch, measured on MI355X per attention call
// (alternating runs, caches cleared before each step): the mixed
// chunked-prefill step 0.1366 against 0.1411 ms, 64 decodes + two 512-token
// chunks 0.294 against 0.311, 128 decodes + four 256-token chunks 0.370
// against 0.392, 8 decodes + one 2048-token chunk 0.2667 against 0.2693.
// The environment variable PKV_MIXED_STEP=fused|split overrides the default.
constexpr bool kFusedStepDefault = true;

bool fused_step() {
    const char* e = std::getenv("PKV_MIXED_STEP");
    if (e && !std::strcmp(e, "fused")) return true;
    if (e && !std::strcmp(e, "split")) return false;
    return kFusedStepDefault;
}

// Of every 4 workgroups of the single launch that carry decode waves and a
// tile, how many run the tile first.  Measured on MI355X per attention call
// (medians of six alternating runs, caches cleared before each step; 0 to 4
// of 4): the mixed chunked-prefill step 0.1366 / 0.1321 / 0.1315 / 0.1369 /
// 0.1440 ms, 64 decodes + two 512-token chunks 0.2735 / 0.2704 / 0.2643 /
// 0.2754 / 0.2960, 8 decodes + one 2048-token chunk 0.2215 / 0.2172 / 0.2170
// / 0.2209 / 0.2266, 16 decodes + two 1024-token chunks 0.2248 / 0.2177 /
// 0.2182 / 0.2257 / 0.2330.  PKV_STEP_TILE_FIRST=0..4 overrides (the output
// is bitwise the same for every value).
constexpr int kStepTileFirstDefault = 2;

int step_tile_first() {
    const char* e = std::getenv("PKV_STEP_TILE_FIRST");
    if (e && e[0] >= '0' && e[0] <= '4' && e[1] == 0) return e[0] - '0';
    return kStepTileFirstDefault;
}

// Whether a decode-only step runs one wave per (sequence, kv head) segment
// (no segment cut, no merge launch) instead of spreading the units evenly
// over kDecodeWaves waves.  Chosen when every segment is short (the host
// bound max_seqlen_k) and there are no more segments than waves: a short
// segment streams in a few page-pair round trips, less than the merge launch
// that cutting it would need.  PKV_DECODE_SEGMENTS=whole|split overrides.
constexpr int kWholeSegmentKeys = 256;

bool whole_segments(int num_seqs, int num_kv_heads, int max_seqlen_k) {
    const bool fits = (long)num_seqs * num_kv_heads <= pkv::kDecodeWaves &&
                      num_seqs <= pkv::kInlinePlanSeqs;
    const char* e = std::getenv("PKV_DECODE_SEGMENTS");
    if (e && !std::strcmp(e, "whole")) return fits;
    if (e && !std::strcmp(e, "split")) return false;
    return fits && max_seqlen_k <= kWholeSegmentKeys;
}

template <typename T, int D>
int launch_prefill(const pkv::PrefillParams& pp, hipStream_t stream, const char* what) {
    const long tiles = prefill_tiles(pp);
    const bool long_ctx = prefill_long<T, D>(pp);
    if (long_ctx)
        hipLaunchKernelGGL((pkv::prefill_kernel<T, D, true>), dim3((unsigned)(tiles * pp.Hkv)),
                           dim3(pkv::PrefillGeom<T, D>::kThreads), 0, stream, pp);
    else
        hipLaunchKernelGGL((pkv::prefill_kernel<T, D, false>), dim3((unsigned)(tiles * pp.Hkv)),
                           dim3(pkv::PrefillGeom<T, D>::kThreads), 0, stream, pp);
    return hip_status(what);
}

template <typename T, int D>
int launch_attention(const pkv::PlanParams& pl, const pkv::DecodeParams& dp,
                     const pkv::MergeParams& mp, const pkv::PrefillParams& pp, int max_seqlen_q,
                     int64_t total_q, int num_seqs, hipStream_t stream) {
    // A step whose host bounds leave no room for a sequence of the decode path
    // runs the prefill launch alone, without a decode pass and a merge that
    // would find nothing to do.  Every sequence has at most max_seqlen_q query
    // tokens and they add up to total_q, so d sequences of at most wmax tokens
    // need num_seqs * max_seqlen_q - total_q >= d * (max_seqlen_q - wmax): a
    // smaller slack means d = 0 (steps of equal-length prefill chunks, for one).
    if (max_seqlen_q > pl.wmax && !dp.prefix_states &&
        (int64_t)num_seqs * max_seqlen_q - total_q < (int64_t)(max_seqlen_q - pl.wmax))
        return launch_prefill<T, D>(pp, stream, "prefill launch");
    // sequences with up to pl.wmax query tokens: plan (large batches only;
    // otherwise each decode wave plans its own pieces), split-key pass, merge
    if (!dp.inline_plan) {
        hipLaunchKernelGGL(pkv::decode_plan_kernel, dim3(1), dim3(pkv::kPlanThreads), 0, stream, pl);
        if (int rc = hip_status("decode plan launch")) return rc;
    }
    if (max_seqlen_q > pl.wmax && !dp.prefix_states && fused_step()) {
        // one launch: every workgroup runs its decode waves and its tile
        pkv::StepParams sp;
        sp.dp = dp;
        sp.pp = pp;
        sp.prefill_wgs = (int)(prefill_tiles(pp) * pp.Hkv);
        constexpr int kWaves = pkv::kStepWaves<T>;
        sp.decode_per_wg = (kWaves < 8 || sp.prefill_wgs >= 2 * pkv::kDecodeWaves / 8) ? 4 : 8;
        sp.decode_wgs = pkv::kDecodeWaves / sp.decode_per_wg;
        sp.tile_first = step_tile_first();
        const unsigned grid = (unsigned)std::max(sp.prefill_wgs, sp.decode_wgs);
        if (prefill_long<T, D>(pp))
            hipLaunchKernelGGL((pkv::step_kernel<T, D, true>), dim3(grid),
                               dim3(pkv::kPrefillThreads<T>), 0, stream, sp);
        else
            hipLaunchKernelGGL((pkv::step_kernel<T, D, false>), dim3(grid),
                               dim3(pkv::kPrefillThreads<T>), 0, stream, sp);
        if (int rc = hip_status("step launch")) return rc;
        hipLaunchKernelGGL((pkv::merge_kernel<T, D>), dim3((unsigned)((long)dp.Hq * num_seqs)),
                           dim3(64), 0, stream, mp);
        return hip_status("merge launch");
    }
    if (dp.whole_segments) {
        // one wave per segment: nothing is cut, so no merge
        hipLaunchKernelGGL((pkv::decode_kernel<T, D, false>),
                           dim3((unsigned)((long)num_seqs * dp.Hkv)), dim3(64), 0, stream, dp);
        return hip_status("decode launch");
    }
    if (dp.prefix_states)
        hipLaunchKernelGGL((pkv::decode_kernel<T, D, true>), dim3(pkv::kDecodeWaves), dim3(64), 0,
                           stream, dp);
    else
        hipLaunchKernelGGL((pkv::decode_kernel<T, D, false>), dim3(pkv::kDecodeWaves), dim3(64), 0,
                           stream, dp);
    if (int rc = hip_status("decode launch")) return rc;
    hipLaunchKernelGGL((pkv::merge_kernel<T, D>), dim3((unsigned)((long)dp.Hq * num_seqs)), dim3(64),
                       0, stream, mp);
    if (int rc = hip_status("merge launch")) return rc;
    if (max_seqlen_q > pl.wmax)  // longer sequences: chunked prefill
        return launch_prefill<T, D>(pp, stream, "prefill launch");
    return PKV_OK;
}

// Shared-prefix steps, ahead of the plain launches: the setup kernel, the
// prefix states of every (group, chunk, kv head) from the prefill kernel, and
// the combination of each member's chunk states when a prefix spans chunks.
template <typename T, int D>
int launch_prefix_pass(const pkv::CascadeParams& cp, const pkv::PrefillParams& spp,
                       const pkv::StateCombineParams& sc, bool combine, hipStream_t stream) {
    hipLaunchKernelGGL(pkv::cascade_setup_kernel, dim3(1), dim3(pkv::kCascadeThreads),
                       pkv::cascade_setup_lds(cp.num_groups), stream, cp);
    if (int rc = hip_status("shared-prefix setup launch")) return rc;
    if (int rc = launch_prefill<T, D>(spp, stream, "shared-prefix state launch")) return rc;
    if (combine) {  // prefixes of more than one chunk
        hipLaunchKernelGGL((pkv::state_combine_kernel<D>), dim3((unsigned)((long)sc.Hq * sc.num_seqs)),
                           dim3(64), 0, stream, sc);
        if (int rc = hip_status("shared-prefix combine launch")) return rc;
    }
    return PKV_OK;
}

// Whether reading each group's prefix once pays for its three extra launches
// (setup, prefix states, combine: ~18 us measured): the K/V re-reads it
// avoids, estimated from the host bounds, against a threshold between the two
// measured cases on MI355X (16 decodes, 40 q / 8 kv heads): a 512-key prefix
// (31 MB avoided; plain path 0.056 ms, prefix pass 0.072 ms) and an 8192-key
// prefix (503 MB avoided; plain 0.075 ms, prefix pass 0.055 ms).
constexpr double kPrefixPassMinSavedBytes = 256.0 * 1024 * 1024;

bool prefix_pass_pays(int num_seqs, int num_groups, int max_group_size, int max_prefix_len,
                      int num_kv_heads, int head_dim, pkv_dtype_t dtype) {
    const double members = std::min(max_group_size, num_seqs);
    if (num_groups <= 0 || members < 2) return false;
    const double saved = (double)num_groups * (members - 1) * max_prefix_len * 2.0 *
                         num_kv_heads * head_dim * (double)elem_bytes(dtype);
    return saved >= kPrefixPassMinSavedBytes;
}

// ------------------------------------------------------- static scratch

// Workspace of pkv_attention_noalloc: a device array of the library's own, so
// that a caller who cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation) needs none.
// Each GPU the library runs on holds its own copy for the life of the process.
// In host code `scratch` names a host-side stand-in, not a device address:
// the device address of a GPU's copy is looked up once per device, with that
// device current, and only that address is ever passed to a kernel.
constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the copy of `scratch` on the GPU that runs `st`.
int scratch_for_stream(hipStream_t st, void** ptr) {
    int dev = -1;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PKV_E_HIP, "device of the stream: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PKV_E_UNSUPPORTED, "device %d: static scratch is kept for devices 0..%d", dev,
                    kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        if (e != hipSuccess) return fail(PKV_E_HIP, "select device %d: %s", dev, hipGetErrorString(e));
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess || !p)
            return fail(PKV_E_HIP, "address of the static scratch on device %d: %s", dev,
                        hipGetErrorString(e));
        if (back != hipSuccess)
            return fail(PKV_E_HIP, "restore device %d: %s", cur, hipGetErrorString(back));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PKV_OK;
}

// Shared-prefix groups of a step (pkv_attention_shared_prefix).
struct PrefixArgs {
    const int32_t* prefix_group;
    const int32_t* prefix_len;
    int num_groups;
    int max_group_size;
    int max_prefix_len;
    bool run_pass;  // false: the step runs as pkv_attention (the workspace is
                    // still checked against the prefix pass's plan)
};

int attention_impl(void* out, const void* q, const void* k_pool, const void* v_pool,
                   const int32_t* block_tables, const int32_t* seq_lens,
                   const int32_t* query_start_loc, const int32_t* kv_start, int num_seqs,
                   int64_t total_q, int max_blocks_per_seq, int max_seqlen_q, int max_seqlen_k,
                   int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                   int64_t num_blocks, float scale, pkv_dtype_t dtype, void* workspace,
                   size_t workspace_bytes, void* stream, const PrefixArgs* pa,
                   bool from_scratch = false) {
    if (int rc = check_common(num_q_heads, num_kv_heads, head_dim, block_size, dtype)) return rc;
    if (num_seqs < 0) return fail(PKV_E_ARG, "num_seqs %d < 0", num_seqs);
    if (total_q < 0) return fail(PKV_E_ARG, "total_q %lld < 0", (long long)total_q);
    if (num_seqs == 0 || total_q == 0) return ok();
    if (!out || !q || !k_pool || !v_pool || !block_tables || !seq_lens || !query_start_loc)
        return fail(PKV_E_ARG, "null pointer argument");
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
        return fail(PKV_E_ARG, "q, out and the pools must be 16-byte aligned");
    if (max_blocks_per_seq <= 0) return fail(PKV_E_ARG, "max_blocks_per_seq %d <= 0", max_blocks_per_seq);
    if (num_blocks <= 0) return fail(PKV_E_ARG, "num_blocks %lld <= 0", (long long)num_blocks);
    if (max_seqlen_q <= 0 || max_seqlen_k <= 0)
        return fail(PKV_E_ARG, "max_seqlen_q %d and max_seqlen_k %d must be positive", max_seqlen_q,
                    max_seqlen_k);
    if (max_seqlen_q > max_seqlen_k)
        return fail(PKV_E_ARG, "max_seqlen_q %d > max_seqlen_k %d", max_seqlen_q, max_seqlen_k);
    if ((int64_t)max_seqlen_k > (int64_t)max_blocks_per_seq * block_size)
        return fail(PKV_E_ARG, "max_seqlen_k %d exceeds the block-table width (%d pages of %d)",
                    max_seqlen_k, max_blocks_per_seq, block_size);
    if (total_q > 0x7fffffffLL) return fail(PKV_E_ARG, "total_q too large");
    // the query counts are at most max_seqlen_q each and add up to total_q
    if (total_q > (int64_t)num_seqs * max_seqlen_q)
        return fail(PKV_E_ARG, "total_q %lld exceeds num_seqs %d x max_seqlen_q %d",
                    (long long)total_q, num_seqs, max_seqlen_q);
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(PKV_E_ARG, "scale %g is not finite and positive", (double)scale);
    const size_t eb = elem_bytes(dtype);
    const size_t io_bytes = (size_t)total_q * num_q_heads * head_dim * eb;
    const size_t pool_bytes = (size_t)num_blocks * num_kv_heads * block_size * head_dim * eb;
    if (overlaps(out, io_bytes, q, io_bytes) || overlaps(out, io_bytes, k_pool, pool_bytes) ||
        overlaps(out, io_bytes, v_pool, pool_bytes))
        return fail(PKV_E_ARG, "out must not alias q or the pools");

    if (num_seqs > pkv::kMaxDecodeSeqs)
        return fail(PKV_E_UNSUPPORTED, "num_seqs %d > %d is not supported", num_seqs,
                    pkv::kMaxDecodeSeqs);
    const int G = num_q_heads / num_kv_heads;
    const Plan pl = make_plan(num_seqs, num_kv_heads, head_dim, G, max_seqlen_q);
    const bool grouped = pa != nullptr && pa->num_groups > 0;
    const bool cascade = grouped && pa->run_pass;
    CascadePlan cpl;
    if (grouped)
        cpl = make_cascade_plan(pl.total, num_seqs, pa->num_groups, pa->max_group_size,
                                pa->max_prefix_len, num_q_heads, num_kv_heads, head_dim);
    const size_t need = grouped ? cpl.total : pl.total;
    if (from_scratch) {
        // every argument is valid: the step runs in the static scratch, if it fits
        if (need > kScratchBytes)
            return fail(PKV_E_WORKSPACE,
                        "the step needs %zu bytes of workspace, above the %zu bytes of static "
                        "scratch (use pkv_attention with a workspace)", need, kScratchBytes);
        if (int rc = scratch_for_stream(static_cast<hipStream_t>(stream), &workspace)) return rc;
        workspace_bytes = kScratchBytes;
    }
    if (!workspace || workspace_bytes < need)
        return fail(PKV_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                    workspace ? workspace_bytes : (size_t)0, need);
    if (!aligned16(workspace)) return fail(PKV_E_ARG, "workspace must be 16-byte aligned");
    if (overlaps(workspace, need, out, io_bytes))
        return fail(PKV_E_ARG, "workspace must not alias out");
    const float scale_log2 = scale * 1.4426950408889634f;
    char* wsb = static_cast<char*>(workspace);
    int32_t* prefix = reinterpret_cast<int32_t*>(wsb + pl.off_prefix);
    int32_t* pbegin = reinterpret_cast<int32_t*>(wsb + pl.off_pbegin);
    pkv::Portion* portions = reinterpret_cast<pkv::Portion*>(wsb + pl.off_portions);
    float* ws_o = reinterpret_cast<float*>(wsb + pl.off_o);
    float* ws_ml = reinterpret_cast<float*>(wsb + pl.off_ml);

    pkv::PlanParams plp{};
    plp.seq_lens = seq_lens;
    plp.qsl = query_start_loc;
    plp.kv_start = kv_start;
    plp.num_seqs = num_seqs;
    plp.Hkv = num_kv_heads;
    plp.max_seqlen_k = max_seqlen_k;
    plp.max_blocks = max_blocks_per_seq;
    plp.wmax = pl.wmax;
    plp.total_q = total_q;
    plp.pair_prefix = prefix;
    plp.portion_begin = pbegin;
    plp.portions = portions;

    pkv::DecodeParams dp{};
    dp.out = out;
    dp.q = q;
    dp.k_pool = k_pool;
    dp.v_pool = v_pool;
    dp.block_tables = block_tables;
    dp.portion_begin = pbegin;
    dp.portions = portions;
    dp.ws_o = ws_o;
    dp.ws_ml = ws_ml;
    dp.max_blocks = max_blocks_per_seq;
    dp.Hq = num_q_heads;
    dp.Hkv = num_kv_heads;
    dp.G = G;
    dp.gmagic = (65536 + G - 1) / G;
    dp.ncol = G * pl.wmax;
    dp.num_blocks = num_blocks;
    dp.inline_plan = num_seqs <= pkv::kInlinePlanSeqs ? 1 : 0;
    dp.seq_lens = seq_lens;
    dp.qsl = query_start_loc;
    dp.kv_start = kv_start;
    dp.num_seqs = num_seqs;
    dp.max_seqlen_k = max_seqlen_k;
    dp.wmax = pl.wmax;
    dp.total_q = total_q;
    dp.pair_prefix = prefix;
    dp.scale_log2 = scale_log2;

    pkv::MergeParams mp{};
    mp.out = out;
    mp.ws_o = ws_o;
    mp.ws_ml = ws_ml;
    mp.pair_prefix = prefix;
    mp.qsl = query_start_loc;
    mp.num_seqs = num_seqs;
    mp.Hq = num_q_heads;
    mp.Hkv = num_kv_heads;
    mp.G = G;
    mp.ncol = G * pl.wmax;

    pkv::PrefillParams pp{};
    pp.out = out;
    pp.q = q;
    pp.k_pool = k_pool;
    pp.v_pool = v_pool;
    pp.block_tables = block_tables;
    pp.seq_lens = seq_lens;
    pp.qsl = query_start_loc;
    pp.kv_start = kv_start;
    pp.num_seqs = num_seqs;
    pp.max_blocks = max_blocks_per_seq;
    pp.Hq = num_q_heads;
    pp.Hkv = num_kv_heads;
    pp.G = G;
    pp.tile_tokens = pl.prefill_tile_tokens;
    pp.min_q = pl.wmax + 1;
    pp.max_seqlen_k = max_seqlen_k;
    pp.total_q = total_q;
    pp.num_blocks = num_blocks;
    pp.scale_log2 = scale_log2;

    hipStream_t st = static_cast<hipStream_t>(stream);
    int rc;
    if (cascade) {
        // the prefix pass's inputs and states live after the plain plan; the
        // plain launches then skip each member's prefix keys (kv_eff) and
        // start its decode segments from the prefix states
        int32_t* kv_eff = reinterpret_cast<int32_t*>(wsb + cpl.off_kv);
        int4* states = reinterpret_cast<int4*>(wsb + cpl.off_states);
        int32_t* v_qsl = reinterpret_cast<int32_t*>(wsb + cpl.off_vqsl);
        int32_t* v_lens = reinterpret_cast<int32_t*>(wsb + cpl.off_vlens);
        int32_t* v_start = reinterpret_cast<int32_t*>(wsb + cpl.off_vstart);
        int32_t* v_row = reinterpret_cast<int32_t*>(wsb + cpl.off_vrow);
        int32_t* v_qrows = reinterpret_cast<int32_t*>(wsb + cpl.off_vqrows);
        float* state = reinterpret_cast<float*>(wsb + cpl.off_state);

        pkv::CascadeParams cp{};
        cp.prefix_group = pa->prefix_group;
        cp.prefix_len = pa->prefix_len;
        cp.qsl = query_start_loc;
        cp.seq_lens = seq_lens;
        cp.num_seqs = num_seqs;
        cp.num_groups = pa->num_groups;
        cp.max_members = pa->max_group_size;
        cp.max_chunks = cpl.max_chunks;
        cp.chunk = cpl.chunk;
        cp.total_q = total_q;
        cp.kv_eff = kv_eff;
        cp.prefix_states = states;
        cp.v_qsl = v_qsl;
        cp.v_lens = v_lens;
        cp.v_start = v_start;
        cp.v_row = v_row;
        cp.v_qrows = v_qrows;

        pkv::PrefillParams spp = pp;
        spp.out = nullptr;
        spp.seq_lens = v_lens;
        spp.qsl = v_qsl;
        spp.kv_start = v_start;
        spp.num_seqs = cpl.V;
        spp.min_q = 1;
        spp.max_seqlen_k = pa->max_prefix_len;
        spp.total_q = cpl.vtokens;
        spp.q_rows = v_qrows;
        spp.seq_row = v_row;
        spp.state = state;
        spp.q_limit = total_q;
        spp.bt_rows = num_seqs;
        spp.sp_tiles = (pa->max_group_size + pp.tile_tokens - 1) / pp.tile_tokens;

        pkv::StateCombineParams sc{};
        sc.prefix_states = states;
        sc.state = state;
        sc.state_rows = cpl.vtokens;
        sc.num_seqs = num_seqs;
        sc.Hq = num_q_heads;

        plp.kv_start = kv_eff;
        dp.kv_start = kv_eff;
        pp.kv_start = kv_eff;
        dp.prefix_states = states;
        dp.state = state;
        dp.state_rows = cpl.vtokens;
        if (dtype == PKV_BF16)
            rc = head_dim == 128 ? launch_prefix_pass<pkv::bf16_t, 128>(cp, spp, sc, cpl.max_chunks > 1, st)
                                 : launch_prefix_pass<pkv::bf16_t, 64>(cp, spp, sc, cpl.max_chunks > 1, st);
        else
            rc = head_dim == 128 ? launch_prefix_pass<float, 128>(cp, spp, sc, cpl.max_chunks > 1, st)
                                 : launch_prefix_pass<float, 64>(cp, spp, sc, cpl.max_chunks > 1, st);
        if (rc) return rc;
    }
    // decode-only steps whose segments are all short: one wave per segment
    dp.whole_segments = (max_seqlen_q <= pl.wmax && !dp.prefix_states &&
                         whole_segments(num_seqs, num_kv_heads, max_seqlen_k)) ? 1 : 0;
    if (dtype == PKV_BF16)
        rc = head_dim == 128 ? launch_attention<pkv::bf16_t, 128>(plp, dp, mp, pp, max_seqlen_q, total_q, num_seqs, st)
                             : launch_attention<pkv::bf16_t, 64>(plp, dp, mp, pp, max_seqlen_q, total_q, num_seqs, st);
    else
        rc = head_dim == 128 ? launch_attention<float, 128>(plp, dp, mp, pp, max_seqlen_q, total_q, num_seqs, st)
                             : launch_attention<float, 64>(plp, dp, mp, pp, max_seqlen_q, total_q, num_seqs, st);
    if (rc) return rc;
    return ok();
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_err.c_str(); }

int pkv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
               const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads, int head_dim,
               int block_size, int64_t num_blocks, pkv_dtype_t dtype, void* stream) {
    if (dtype != PKV_F32 && dtype != PKV_BF16)
        return fail(PKV_E_UNSUPPORTED, "dtype %d is not supported", (int)dtype);
    if (num_tokens < 0) return fail(PKV_E_ARG, "num_tokens %lld < 0", (long long)num_tokens);
    if (num_kv_heads <= 0) return fail(PKV_E_ARG, "num_kv_heads %d <= 0", num_kv_heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(PKV_E_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", head_dim);
    if (block_size < 1 || block_size > 256)
        return fail(PKV_E_UNSUPPORTED, "block_size %d outside [1, 256]", block_size);
    if (num_blocks <= 0) return fail(PKV_E_ARG, "num_blocks %lld <= 0", (long long)num_blocks);
    if (num_tokens == 0) return ok();
    if (!k_new || !v_new || !k_pool || !v_pool || !slot_mapping)
        return fail(PKV_E_ARG, "null pointer argument");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
        return fail(PKV_E_ARG, "K/V buffers must be 16-byte aligned");
    const size_t rb = (size_t)head_dim * elem_bytes(dtype);
    const size_t pool_bytes = (size_t)num_blocks * num_kv_heads * block_size * rb;
    const size_t new_bytes = (size_t)num_tokens * num_kv_heads * rb;
    if (overlaps(k_new, new_bytes, k_pool, pool_bytes) || overlaps(v_new, new_bytes, v_pool, pool_bytes) ||
        overlaps(k_pool, pool_bytes, v_pool, pool_bytes))
        return fail(PKV_E_ARG, "new rows and pools must not overlap");
    pkv::AppendParams ap;
    ap.k_new = static_cast<const uint8_t*>(k_new);
    ap.v_new = static_cast<const uint8_t*>(v_new);
    ap.k_pool = static_cast<uint8_t*>(k_pool);
    ap.v_pool = static_cast<uint8_t*>(v_pool);
    ap.slots = slot_mapping;
    ap.rows = num_tokens * num_kv_heads;
    ap.num_kv_heads = num_kv_heads;
    ap.chunks_per_row = (int)(rb / 16);
    ap.block_size = block_size;
    ap.num_slots = num_blocks * block_size;
    const int64_t threads = ap.rows * ap.chunks_per_row;
    const int64_t grid = (threads + 255) / 256;
    if (grid > 0x7fffffffLL) return fail(PKV_E_ARG, "too many tokens for one launch");
    hipLaunchKernelGGL(pkv::append_kernel, dim3((unsigned)grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), ap);
    if (int rc = hip_status("append launch")) return rc;
    return ok();
}

size_t pkv_attention_workspace_size(int num_seqs, int64_t total_q, int max_seqlen_q,
                                    int max_seqlen_k, int num_q_heads, int num_kv_heads,
                                    int head_dim, int block_size, pkv_dtype_t dtype) {
    (void)total_q;
    (void)max_seqlen_k;
    (void)dtype;
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size != kBlock || num_q_heads % num_kv_heads)
        return 0;
    return make_plan(num_seqs, num_kv_heads, head_dim, num_q_heads / num_kv_heads,
                     std::max(1, max_seqlen_q)).total;
}

int pkv_attention(void* out, const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* block_tables, const int32_t* seq_lens,
                  const int32_t* query_start_loc, const int32_t* kv_start, int num_seqs,
                  int64_t total_q, int max_blocks_per_seq, int max_seqlen_q, int max_seqlen_k,
                  int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                  int64_t num_blocks, float scale, pkv_dtype_t dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
    return attention_impl(out, q, k_pool, v_pool, block_tables, seq_lens, query_start_loc,
                          kv_start, num_seqs, total_q, max_blocks_per_seq, max_seqlen_q,
                          max_seqlen_k, num_q_heads, num_kv_heads, head_dim, block_size,
                          num_blocks, scale, dtype, workspace, workspace_bytes, stream, nullptr);
}

int pkv_attention_noalloc(void* out, const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* seq_lens,
                          const int32_t* query_start_loc, const int32_t* kv_start, int num_seqs,
                          int64_t total_q, int max_blocks_per_seq, int max_seqlen_q,
                          int max_seqlen_k, int num_q_heads, int num_kv_heads, int head_dim,
                          int block_size, int64_t num_blocks, float scale, pkv_dtype_t dtype,
                          void* stream) {
    return attention_impl(out, q, k_pool, v_pool, block_tables, seq_lens, query_start_loc,
                          kv_start, num_seqs, total_q, max_blocks_per_seq, max_seqlen_q,
                          max_seqlen_k, num_q_heads, num_kv_heads, head_dim, block_size,
                          num_blocks, scale, dtype, nullptr, 0, stream, nullptr, true);
}

size_t pkv_attention_shared_prefix_workspace_size(int num_seqs, int64_t total_q, int max_seqlen_q,
                                                  int max_seqlen_k, int num_q_heads,
                                                  int num_kv_heads, int head_dim, int block_size,
                                                  pkv_dtype_t dtype, int num_groups,
                                                  int max_group_size, int max_prefix_len) {
    const size_t base = pkv_attention_workspace_size(num_seqs, total_q, max_seqlen_q, max_seqlen_k,
                                                     num_q_heads, num_kv_heads, head_dim,
                                                     block_size, dtype);
    if (base == 0 || num_groups <= 0 || max_group_size <= 0 || max_prefix_len <= 0) return base;
    return make_cascade_plan(base, num_seqs, num_groups, max_group_size, max_prefix_len,
                             num_q_heads, num_kv_heads, head_dim).total;
}

int pkv_attention_shared_prefix(void* out, const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                const int32_t* query_start_loc, const int32_t* prefix_group,
                                const int32_t* prefix_len, int num_groups, int max_group_size,
                                int max_prefix_len, int num_seqs, int64_t total_q,
                                int max_blocks_per_seq, int max_seqlen_q, int max_seqlen_k,
                                int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                int64_t num_blocks, float scale, pkv_dtype_t dtype,
                                int prefix_pass, void* workspace, size_t workspace_bytes,
                                void* stream) {
    // head counts, head_dim, block_size and dtype first: the prefix checks
    // below divide by block_size
    if (int rc = check_common(num_q_heads, num_kv_heads, head_dim, block_size, dtype)) return rc;
    if (num_groups < 0) return fail(PKV_E_ARG, "num_groups %d < 0", num_groups);
    if (num_groups > pkv::kCascadeMaxGroups)
        return fail(PKV_E_UNSUPPORTED, "num_groups %d > %d is not supported", num_groups,
                    pkv::kCascadeMaxGroups);
    PrefixArgs pa{prefix_group, prefix_len, num_groups, max_group_size, max_prefix_len, true};
    if (num_groups > 0 && num_seqs > 0 && total_q > 0) {
        if (!prefix_group || !prefix_len) return fail(PKV_E_ARG, "null pointer argument");
        if (max_group_size <= 0)
            return fail(PKV_E_ARG, "max_group_size %d must be positive", max_group_size);
        if (max_prefix_len <= 0 || max_prefix_len % block_size)
            return fail(PKV_E_ARG, "max_prefix_len %d must be a positive multiple of block_size %d",
                        max_prefix_len, block_size);
        if (max_prefix_len >= max_seqlen_k)
            return fail(PKV_E_ARG, "max_prefix_len %d must be below max_seqlen_k %d",
                        max_prefix_len, max_seqlen_k);
    }
    if (prefix_pass != PKV_PREFIX_PASS_AUTO && prefix_pass != PKV_PREFIX_PASS_ALWAYS)
        return fail(PKV_E_ARG, "prefix_pass %d is neither AUTO nor ALWAYS", prefix_pass);
    pa.run_pass = prefix_pass == PKV_PREFIX_PASS_ALWAYS ||
                  prefix_pass_pays(num_seqs, num_groups, max_group_size, max_prefix_len,
                                   num_kv_heads, head_dim, dtype);
    return attention_impl(out, q, k_pool, v_pool, block_tables, seq_lens, query_start_loc,
                          nullptr, num_seqs, total_q, max_blocks_per_seq, max_seqlen_q,
                          max_seqlen_k, num_q_heads, num_kv_heads, head_dim, block_size,
                          num_blocks, scale, dtype, workspace, workspace_bytes, stream, &pa);
}

int pkv_check_metadata(const int32_t* block_tables, const int32_t* seq_lens,
                       const int32_t* query_start_loc, const int32_t* kv_start, int num_seqs,
                       int64_t total_q, int max_blocks_per_seq, int max_seqlen_q,
                       int max_seqlen_k, int block_size, int64_t num_blocks) {
    if (num_seqs < 0 || block_size <= 0 || max_blocks_per_seq < 0 || num_blocks < 0 ||
        max_seqlen_q < 0 || max_seqlen_k < 0)
        return fail(PKV_E_ARG, "invalid sizes");
    if (num_seqs == 0) return ok();
    if (!block_tables || !seq_lens || !query_start_loc)
        return fail(PKV_E_ARG, "null pointer argument");
    if (query_start_loc[0] != 0) return fail(PKV_E_METADATA, "query_start_loc[0] = %d, not 0", query_start_loc[0]);
    if (query_start_loc[num_seqs] != total_q)
        return fail(PKV_E_METADATA, "query_start_loc[%d] = %d, not total_q %lld", num_seqs,
                    query_start_loc[num_seqs], (long long)total_q);
    for (int s = 0; s < num_seqs; ++s) {
        const int64_t n = (int64_t)query_start_loc[s + 1] - query_start_loc[s];
        const int64_t L = seq_lens[s];
        const int64_t a = kv_start ? kv_start[s] : 0;
        if (n < 0) return fail(PKV_E_METADATA, "query_start_loc decreases at sequence %d", s);
        if (L < 0) return fail(PKV_E_METADATA, "seq_lens[%d] = %lld < 0", s, (long long)L);
        if (a < 0 || a > L)
            return fail(PKV_E_METADATA, "kv_start[%d] = %lld outside [0, %lld]", s, (long long)a, (long long)L);
        if (n > L - a)
            return fail(PKV_E_METADATA, "sequence %d has %lld query tokens but %lld visible keys", s,
                        (long long)n, (long long)(L - a));
        if (n > max_seqlen_q)
            return fail(PKV_E_METADATA, "sequence %d has %lld query tokens, above max_seqlen_q %d",
                        s, (long long)n, max_seqlen_q);
        if (L > max_seqlen_k)
            return fail(PKV_E_METADATA, "seq_lens[%d] = %lld is above max_seqlen_k %d", s,
                        (long long)L, max_seqlen_k);
        if (L == 0) continue;
        const int64_t last = (L - 1) / block_size;
        if (last >= max_blocks_per_seq)
            return fail(PKV_E_METADATA, "sequence %d needs %lld pages, block table has %d", s,
                        (long long)(last + 1), max_blocks_per_seq);
        for (int64_t pg = a / block_size; pg <= last; ++pg) {
            const int32_t b = block_tables[(int64_t)s * max_blocks_per_seq + pg];
            if (b < 0 || b >= num_blocks)
                return fail(PKV_E_METADATA, "block_tables[%d][%lld] = %d outside [0, %lld)", s,
                            (long long)pg, b, (long long)num_blocks);
        }
    }
    return ok();
}

int pkv_check_shared_prefix(const int32_t* block_tables, const int32_t* seq_lens,
                            const int32_t* query_start_loc, const int32_t* prefix_group,
                            const int32_t* prefix_len, int num_seqs, int num_groups,
                            int max_blocks_per_seq, int block_size, int max_prefix_len) {
    if (num_seqs < 0 || num_groups < 0 || max_blocks_per_seq < 0 || block_size <= 0)
        return fail(PKV_E_ARG, "invalid sizes");
    if (num_seqs == 0 || num_groups == 0) return ok();
    if (!block_tables || !seq_lens || !query_start_loc || !prefix_group || !prefix_len)
        return fail(PKV_E_ARG, "null pointer argument");
    std::vector<int> first(num_groups, -1);
    for (int g = 0; g < num_groups; ++g) {
        const int P = prefix_len[g];
        if (P < 0 || P % block_size || P > max_prefix_len)
            return fail(PKV_E_METADATA, "prefix_len[%d] = %d is not a multiple of %d in [0, %d]", g,
                        P, block_size, max_prefix_len);
        if (P / block_size > max_blocks_per_seq)
            return fail(PKV_E_METADATA, "prefix_len[%d] = %d exceeds the block-table width", g, P);
    }
    for (int s = 0; s < num_seqs; ++s) {
        const int g = prefix_group[s];
        if (g == -1) continue;
        if (g < 0 || g >= num_groups)
            return fail(PKV_E_METADATA, "prefix_group[%d] = %d outside [-1, %d)", s, g, num_groups);
        const int n = query_start_loc[s + 1] - query_start_loc[s];
        if (n != 1)
            return fail(PKV_E_METADATA, "sequence %d of group %d has %d query tokens, not 1", s, g, n);
        if (seq_lens[s] <= prefix_len[g])
            return fail(PKV_E_METADATA, "sequence %d has %d keys, not more than its prefix of %d",
                        s, seq_lens[s], prefix_len[g]);
        if (first[g] < 0) {
            first[g] = s;
            continue;
        }
        const int32_t* a = block_tables + (int64_t)first[g] * max_blocks_per_seq;
        const int32_t* b = block_tables + (int64_t)s * max_blocks_per_seq;
        for (int pg = 0; pg < prefix_len[g] / block_size; ++pg)
            if (a[pg] != b[pg])
                return fail(PKV_E_METADATA,
                            "sequences %d and %d of group %d differ at prefix page %d (%d, %d)",
                            first[g], s, g, pg, a[pg], b[pg]);
    }
    return ok();
}

int pkv_check_slots(const int64_t* slot_mapping, int64_t num_tokens, int block_size,
                    int64_t num_blocks) {
    if (num_tokens < 0 || block_size <= 0 || num_blocks < 0) return fail(PKV_E_ARG, "invalid sizes");
    if (num_tokens == 0) return ok();
    if (!slot_mapping) return fail(PKV_E_ARG, "null pointer argument");
    const int64_t nslots = num_blocks * block_size;
    std::vector<int64_t> seen;
    seen.reserve((size_t)num_tokens);
    for (int64_t t = 0; t < num_tokens; ++t) {
        const int64_t v = slot_mapping[t];
        if (v < 0) continue;
        if (v >= nslots)
            return fail(PKV_E_METADATA, "slot_mapping[%lld] = %lld outside [0, %lld)", (long long)t,
                        (long long)v, (long long)nslots);
        seen.push_back(v);
    }
    std::sort(seen.begin(), seen.end());
    for (size_t i = 1; i < seen.size(); ++i)
        if (seen[i] == seen[i - 1])
            return fail(PKV_E_METADATA, "slot %lld is written twice", (long long)seen[i]);
    return ok();
}


// ---------------------------------------------------------------- pool manager

pkv_pool_t* pkv_pool_create(int64_t num_blocks, int block_size, int max_seqs,
                            int max_blocks_per_seq) {
    if (num_blocks <= 0 || num_blocks > 0x7fffffffLL || block_size <= 0 || max_seqs <= 0 ||
        max_blocks_per_seq <= 0) {
        fail(PKV_E_ARG, "invalid pool sizes");
        return nullptr;
    }
    try {
        pkv_pool_t* p = new pkv_pool_t{pkv::PagePool(num_blocks, block_size, max_seqs,
                                                     max_blocks_per_seq)};
        ok();
        return p;
    } catch (...) {
        fail(PKV_E_ARG, "host allocation of the pool tables failed");
        return nullptr;
    }
}

void pkv_pool_destroy(pkv_pool_t* pool) { delete pool; }

int64_t pkv_pool_free_blocks(const pkv_pool_t* pool) {
    return pool ? pool->pool.free_blocks() : -1;
}

int pkv_pool_set_free_order(pkv_pool_t* pool, const int32_t* order, int64_t n) {
    if (!pool) return fail(PKV_E_ARG, "null pool");
    if (pool->pool.set_free_order(order, n) != pkv::PagePool::kOk)
        return fail(PKV_E_ARG, "the order must list each of the %lld free pages once",
                    (long long)pool->pool.free_blocks());
    return ok();
}

int pkv_pool_can_admit(const pkv_pool_t* pool, int64_t num_tokens) {
    return pool ? (pool->pool.can_admit(num_tokens) ? 1 : 0) : -1;
}

static int pool_status(pkv::PagePool::Status st, const char* what) {
    switch (st) {
    case pkv::PagePool::kOk: return ok();
    case pkv::PagePool::kNoMem: return fail(PKV_E_NOMEM, "%s: too few free pages", what);
    default: return fail(PKV_E_ARG, "%s: invalid sequence or size", what);
    }
}

int pkv_pool_add_seq(pkv_pool_t* pool, int seq) {
    if (!pool) return fail(PKV_E_ARG, "null pool");
    return pool_status(pool->pool.add_seq(seq), "pkv_pool_add_seq");
}

int pkv_pool_fork(pkv_pool_t* pool, int parent, int child, int64_t shared_tokens) {
    if (!pool) return fail(PKV_E_ARG, "null pool");
    return pool_status(pool->pool.fork(parent, child, shared_tokens), "pkv_pool_fork");
}

int pkv_pool_append(pkv_pool_t* pool, int seq, int64_t num_tokens, int64_t* slots,
                    int32_t* cow_src, int32_t* cow_dst, int* num_cow) {
    if (!pool) return fail(PKV_E_ARG, "null pool");
    if (num_tokens > 0 && !slots) return fail(PKV_E_ARG, "null slots");
    pkv::PagePool& pp = pool->pool;
    if (pp.live(seq) && num_tokens > 0 && pp.length(seq) % pp.block_size() != 0 &&
        pp.refcount(pp.pages(seq).back()) > 1 && (!cow_src || !cow_dst || !num_cow))
        return fail(PKV_E_ARG, "pkv_pool_append: a page copy is needed but cow outputs are NULL");
    return pool_status(pp.append(seq, num_tokens, slots, cow_src, cow_dst, num_cow),
                       "pkv_pool_append");
}

int pkv_pool_append_batch(pkv_pool_t* pool, const int* seqs, const int64_t* counts,
                          int num_seqs, int64_t* slots, int32_t* cow_src, int32_t* cow_dst,
                          int* num_cow) {
    if (!pool) return fail(PKV_E_ARG, "null pool");
    if (num_seqs < 0) return fail(PKV_E_ARG, "num_seqs %d < 0", num_seqs);
    if (num_seqs == 0) {
        if (num_cow) *num_cow = 0;
        return ok();
    }
    if (!seqs || !counts || !slots || !cow_src || !cow_dst || !num_cow)
        return fail(PKV_E_ARG, "null pointer argument");
    return pool_status(pool->pool.append_batch(seqs, counts, num_seqs, slots, cow_src, cow_dst,
                                               num_cow),
                       "pkv_pool_append_batch");
}

int pkv_pool_truncate(pkv_pool_t* pool, int seq, int64_t new_len) {
    if (!pool) return fail(PKV_E_ARG, "null pool");
    return pool_status(pool->pool.truncate(seq, new_len), "pkv_pool_truncate");
}

int pkv_pool_free_seq(pkv_pool_t* pool, int seq) {
    if (!pool) return fail(PKV_E_ARG, "null pool");
    return pool_status(pool->pool.free_seq(seq), "pkv_pool_free_seq");
}

int64_t pkv_pool_seq_len(const pkv_pool_t* pool, int seq) {
    return pool ? pool->pool.length(seq) : -1;
}

int pkv_pool_block_tables(const pkv_pool_t* pool, const int* seqs, int num_seqs, int32_t* table,
                          int width, int32_t* seq_lens) {
    if (!pool) return fail(PKV_E_ARG, "null pool");
    if (num_seqs < 0 || width <= 0) return fail(PKV_E_ARG, "invalid sizes");
    if (num_seqs == 0) return ok();
    if (!seqs || !table) return fail(PKV_E_ARG, "null pointer argument");
    const pkv::PagePool& pp = pool->pool;
    for (int i = 0; i < num_seqs; ++i) {
        if (!pp.live(seqs[i])) return fail(PKV_E_ARG, "sequence %d is not live", seqs[i]);
        if ((int64_t)pp.pages(seqs[i]).size() > width)
            return fail(PKV_E_ARG, "sequence %d holds %zu pages, table width %d", seqs[i],
                        pp.pages(seqs[i]).size(), width);
    }
    for (int i = 0; i < num_seqs; ++i) {
        const std::vector<int32_t>& pg = pp.pages(seqs[i]);
        int32_t* row = table + (int64_t)i * width;
        for (int j = 0; j < width; ++j) row[j] = j < (int)pg.size() ? pg[(size_t)j] : -1;
        if (seq_lens) seq_lens[i] = (int32_t)pp.length(seqs[i]);
    }
    return ok();
}

int pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst,
                    int64_t num_pairs, int num_kv_heads, int head_dim, int block_size,
                    int64_t num_blocks, pkv_dtype_t dtype, void* stream) {
    if (dtype != PKV_F32 && dtype != PKV_BF16)
        return fail(PKV_E_UNSUPPORTED, "dtype %d is not supported", (int)dtype);
    if (num_pairs < 0) return fail(PKV_E_ARG, "num_pairs %lld < 0", (long long)num_pairs);
    if (num_kv_heads <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PKV_E_ARG, "invalid sizes");
    if (head_dim != 64 && head_dim != 128)
        return fail(PKV_E_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", head_dim);
    if (num_pairs == 0) return ok();
    if (!k_pool || !v_pool || !src || !dst) return fail(PKV_E_ARG, "null pointer argument");
    if (!aligned16(k_pool) || !aligned16(v_pool))
        return fail(PKV_E_ARG, "pools must be 16-byte aligned");
    pkv::CopyBlocksParams cp;
    cp.k_pool = static_cast<uint8_t*>(k_pool);
    cp.v_pool = static_cast<uint8_t*>(v_pool);
    cp.src = src;
    cp.dst = dst;
    cp.num_pairs = num_pairs;
    cp.chunks_per_block = (int64_t)num_kv_heads * block_size * head_dim * (int64_t)elem_bytes(dtype) / 16;
    cp.num_blocks = num_blocks;
    const int64_t grid = (num_pairs * cp.chunks_per_block + 255) / 256;
    if (grid > 0x7fffffffLL) return fail(PKV_E_ARG, "too many pages for one launch");
    hipLaunchKernelGGL(pkv::copy_blocks_kernel, dim3((unsigned)grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), cp);
    if (int rc = hip_status("copy launch")) return rc;
    return ok();
}

}  // extern "C"
