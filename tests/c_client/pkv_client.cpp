// A plain C++ caller of the library's C ABI: HIP runtime calls and libpkv.so
// only (no Python, no torch).  It fills a paged pool with pkv_append, runs
// pkv_attention on one packed step (two decodes, a 3-token verify window and a
// 40-token prefill chunk; 8 query / 2 kv heads, head_dim 128; pages shuffled
// over the pool; unused pool bytes NaN), checks the pool bytes and the output
// against the float64 oracle (linked from oracle/, test infrastructure), and
// checks that invalid calls fail with their documented codes and launch
// nothing.  Exit status 0 when every check passes.
//
// Built by __graft_entry__.build(); run by tests/test_c_client.py.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "pkv.h"

extern "C" {
// float64 oracle (oracle/pkv_oracle.c)
int oracle_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                  const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                  int head_dim, int block_size, int64_t num_blocks, int dtype);
int oracle_attention(double* out, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, const int32_t* seq_lens,
                     const int32_t* query_start_loc, const int32_t* kv_start, int num_seqs,
                     int max_blocks_per_seq, int num_q_heads, int num_kv_heads, int head_dim,
                     int block_size, int64_t num_blocks, double scale, int dtype,
                     int num_threads);
}

namespace {

int g_failures = 0;

void check(bool ok, const char* what) {
    if (!ok) {
        std::printf("FAIL: %s\n", what);
        ++g_failures;
    }
}

#define HIP_OK(call)                                                                   \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            std::printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__,  \
                        __LINE__);                                                     \
            return 2;                                                                  \
        }                                                                              \
    } while (0)

// splitmix64: a counter-based generator, the same stream on every host
struct Rng {
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9e3779b97f4a7c15ull);
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        return z ^ (z >> 31);
    }
    double uniform() { return (double)(next() >> 11) * (1.0 / 9007199254740992.0); }
    // approximately N(0, 1): sum of four uniforms, centred and scaled
    float normal() {
        double a = uniform() + uniform() + uniform() + uniform() - 2.0;
        return (float)(a * 1.7320508075688772);
    }
};

uint16_t to_bf16(float f) {  // round to nearest even (finite inputs)
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float from_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

int run_case(pkv_dtype_t dtype) {
    const bool bf = dtype == PKV_BF16;
    const size_t eb = bf ? 2 : 4;
    const int Hq = 8, Hkv = 2, D = 128, BS = 16;
    const std::vector<int> lens = {37, 300, 129, 1000};
    const std::vector<int> nq = {1, 1, 40, 3};
    const int S = (int)lens.size();
    Rng rng{bf ? 11u : 12u};

    // block tables over a shuffled pool of 1.25x the pages needed
    int need = 0, max_blocks = 0;
    for (int L : lens) {
        need += (L + BS - 1) / BS;
        max_blocks = std::max(max_blocks, (L + BS - 1) / BS);
    }
    const int64_t num_blocks = need + need / 4;
    std::vector<int32_t> perm(num_blocks);
    for (int64_t i = 0; i < num_blocks; ++i) perm[i] = (int32_t)i;
    for (int64_t i = num_blocks - 1; i > 0; --i) std::swap(perm[i], perm[rng.next() % (i + 1)]);
    std::vector<int32_t> bt((size_t)S * max_blocks, -1);
    int used = 0;
    for (int s = 0; s < S; ++s)
        for (int pg = 0; pg < (lens[s] + BS - 1) / BS; ++pg) bt[(size_t)s * max_blocks + pg] = perm[used++];

    // every key of every sequence, appended in one call
    int64_t T = 0;
    for (int L : lens) T += L;
    const size_t row = (size_t)Hkv * D;
    std::vector<uint8_t> knew(T * row * eb), vnew(T * row * eb);
    std::vector<int64_t> slots(T);
    int64_t t = 0;
    for (int s = 0; s < S; ++s)
        for (int j = 0; j < lens[s]; ++j, ++t) {
            slots[t] = (int64_t)bt[(size_t)s * max_blocks + j / BS] * BS + j % BS;
            for (size_t e = 0; e < row; ++e) {
                const float kf = rng.normal(), vf = rng.normal();
                if (bf) {
                    reinterpret_cast<uint16_t*>(knew.data())[t * row + e] = to_bf16(kf);
                    reinterpret_cast<uint16_t*>(vnew.data())[t * row + e] = to_bf16(vf);
                } else {
                    reinterpret_cast<float*>(knew.data())[t * row + e] = kf;
                    reinterpret_cast<float*>(vnew.data())[t * row + e] = vf;
                }
            }
        }
    const size_t pool_bytes = (size_t)num_blocks * Hkv * BS * D * eb;
    std::vector<uint8_t> kpool_ref(pool_bytes, 0xff), vpool_ref(pool_bytes, 0xff);  // NaN bytes
    check(oracle_append(kpool_ref.data(), vpool_ref.data(), knew.data(), vnew.data(), slots.data(),
                        T, Hkv, D, BS, num_blocks, bf ? 1 : 0) == 0,
          "oracle append");

    // the step
    std::vector<int32_t> qsl(S + 1, 0);
    for (int s = 0; s < S; ++s) qsl[s + 1] = qsl[s] + nq[s];
    const int64_t total_q = qsl[S];
    int max_q = 0, max_k = 0;
    for (int s = 0; s < S; ++s) {
        max_q = std::max(max_q, nq[s]);
        max_k = std::max(max_k, lens[s]);
    }
    std::vector<uint8_t> q((size_t)total_q * Hq * D * eb);
    for (size_t e = 0; e < (size_t)total_q * Hq * D; ++e) {
        const float f = rng.normal();
        if (bf) reinterpret_cast<uint16_t*>(q.data())[e] = to_bf16(f);
        else reinterpret_cast<float*>(q.data())[e] = f;
    }
    const float scale = 1.0f / std::sqrt((float)D);

    // device side: caller-owned buffers, one stream
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    void *d_kpool, *d_vpool, *d_knew, *d_vnew, *d_slots, *d_q, *d_out, *d_bt, *d_lens, *d_qsl;
    HIP_OK(hipMalloc(&d_kpool, pool_bytes));
    HIP_OK(hipMalloc(&d_vpool, pool_bytes));
    HIP_OK(hipMemset(d_kpool, 0xff, pool_bytes));
    HIP_OK(hipMemset(d_vpool, 0xff, pool_bytes));
    HIP_OK(hipMalloc(&d_knew, knew.size()));
    HIP_OK(hipMalloc(&d_vnew, vnew.size()));
    HIP_OK(hipMalloc(&d_slots, slots.size() * 8));
    HIP_OK(hipMalloc(&d_q, q.size()));
    HIP_OK(hipMalloc(&d_out, q.size()));
    HIP_OK(hipMalloc(&d_bt, bt.size() * 4));
    HIP_OK(hipMalloc(&d_lens, S * 4));
    HIP_OK(hipMalloc(&d_qsl, (S + 1) * 4));
    HIP_OK(hipMemcpy(d_knew, knew.data(), knew.size(), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_vnew, vnew.data(), vnew.size(), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_slots, slots.data(), slots.size() * 8, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_q, q.data(), q.size(), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_bt, bt.data(), bt.size() * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_lens, lens.data(), S * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_qsl, qsl.data(), (S + 1) * 4, hipMemcpyHostToDevice));

    check(pkv_check_slots(slots.data(), T, BS, num_blocks) == PKV_OK, "pkv_check_slots");
    check(pkv_check_metadata(bt.data(), lens.data(), qsl.data(), nullptr, S, total_q, max_blocks,
                             max_q, max_k, BS, num_blocks) == PKV_OK,
          "pkv_check_metadata");
    check(pkv_check_metadata(bt.data(), lens.data(), qsl.data(), nullptr, S, total_q, max_blocks,
                             max_q - 1, max_k, BS, num_blocks) == PKV_E_METADATA,
          "pkv_check_metadata rejects an understated max_seqlen_q");
    int rc = pkv_append(d_knew, d_vnew, d_kpool, d_vpool, (const int64_t*)d_slots, T, Hkv, D, BS,
                        num_blocks, dtype, stream);
    check(rc == PKV_OK, "pkv_append");
    const size_t ws = pkv_attention_workspace_size(S, total_q, max_q, max_k, Hq, Hkv, D, BS, dtype);
    void* d_ws = nullptr;
    if (ws) HIP_OK(hipMalloc(&d_ws, ws));
    rc = pkv_attention(d_out, d_q, d_kpool, d_vpool, (const int32_t*)d_bt, (const int32_t*)d_lens,
                       (const int32_t*)d_qsl, nullptr, S, total_q, max_blocks, max_q, max_k, Hq,
                       Hkv, D, BS, num_blocks, scale, dtype, d_ws, ws, stream);
    check(rc == PKV_OK, "pkv_attention");
    if (rc != PKV_OK) std::printf("  %s\n", pkv_last_error());

    // invalid calls: documented codes, a reason, and nothing launched
    HIP_OK(hipStreamSynchronize(stream));
    std::vector<uint8_t> out_before(q.size());
    HIP_OK(hipMemcpy(out_before.data(), d_out, q.size(), hipMemcpyDeviceToHost));
    HIP_OK(hipMemset(d_out, 0, q.size()));
    rc = pkv_attention(d_out, d_q, d_kpool, d_vpool, (const int32_t*)d_bt, (const int32_t*)d_lens,
                       (const int32_t*)d_qsl, nullptr, S, total_q, max_blocks, max_q, max_k, Hq,
                       Hkv, D, BS, num_blocks, 0.0f, dtype, d_ws, ws, stream);
    check(rc == PKV_E_ARG && std::strlen(pkv_last_error()) > 0, "scale 0 is PKV_E_ARG");
    rc = pkv_attention(d_out, d_q, d_kpool, d_vpool, (const int32_t*)d_bt, (const int32_t*)d_lens,
                       (const int32_t*)d_qsl, nullptr, S, total_q, max_blocks, max_q, max_k, Hq,
                       Hkv, 96, BS, num_blocks, scale, dtype, d_ws, ws, stream);
    check(rc == PKV_E_UNSUPPORTED, "head_dim 96 is PKV_E_UNSUPPORTED");
    if (ws) {
        rc = pkv_attention(d_out, d_q, d_kpool, d_vpool, (const int32_t*)d_bt,
                           (const int32_t*)d_lens, (const int32_t*)d_qsl, nullptr, S, total_q,
                           max_blocks, max_q, max_k, Hq, Hkv, D, BS, num_blocks, scale, dtype,
                           d_ws, ws - 1, stream);
        check(rc == PKV_E_WORKSPACE, "short workspace is PKV_E_WORKSPACE");
    }
    rc = pkv_append(d_knew, d_vnew, d_kpool, d_vpool, (const int64_t*)d_slots, T, 0, D, BS,
                    num_blocks, dtype, stream);
    check(rc == PKV_E_ARG, "num_kv_heads 0 is PKV_E_ARG");
    rc = pkv_append(d_knew, d_vnew, d_kpool, d_vpool, (const int64_t*)d_slots, T, Hkv, D, 0,
                    num_blocks, dtype, stream);
    check(rc == PKV_E_UNSUPPORTED, "block_size 0 is PKV_E_UNSUPPORTED");
    HIP_OK(hipStreamSynchronize(stream));
    std::vector<uint8_t> out_after(q.size());
    HIP_OK(hipMemcpy(out_after.data(), d_out, q.size(), hipMemcpyDeviceToHost));
    bool untouched = true;
    for (uint8_t b : out_after) untouched = untouched && b == 0;
    check(untouched, "invalid calls launch nothing");

    // pool bytes and output against the oracle
    std::vector<uint8_t> kpool(pool_bytes), vpool(pool_bytes);
    HIP_OK(hipMemcpy(kpool.data(), d_kpool, pool_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(vpool.data(), d_vpool, pool_bytes, hipMemcpyDeviceToHost));
    check(kpool == kpool_ref && vpool == vpool_ref, "pool bytes equal the oracle append");
    std::vector<double> ref((size_t)total_q * Hq * D);
    check(oracle_attention(ref.data(), q.data(), kpool_ref.data(), vpool_ref.data(), bt.data(),
                           lens.data(), qsl.data(), nullptr, S, max_blocks, Hq, Hkv, D, BS,
                           num_blocks, (double)scale, bf ? 1 : 0, 0) == 0,
          "oracle attention");
    const double tol = bf ? 1e-2 : 1e-5;
    double max_err = 0.0;
    size_t bad = 0;
    for (size_t e = 0; e < ref.size(); ++e) {
        const double g = bf ? (double)from_bf16(reinterpret_cast<uint16_t*>(out_before.data())[e])
                            : (double)reinterpret_cast<float*>(out_before.data())[e];
        const double err = std::fabs(g - ref[e]);
        if (!(err <= tol + tol * std::fabs(ref[e]))) ++bad;
        if (!(err <= max_err)) max_err = err;
    }
    check(bad == 0, "attention within tolerance of the oracle");
    std::printf("%s: %lld query tokens, %lld keys, max |err| %.3e (tol %.0e), %zu outside\n",
                bf ? "bf16" : "fp32", (long long)total_q, (long long)T, max_err, tol, bad);

    for (void* ptr : {d_kpool, d_vpool, d_knew, d_vnew, d_slots, d_q, d_out, d_bt, d_lens, d_qsl})
        HIP_OK(hipFree(ptr));
    if (d_ws) HIP_OK(hipFree(d_ws));
    HIP_OK(hipStreamDestroy(stream));
    return 0;
}

}  // namespace

int main() {
    int dev_count = 0;
    if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count < 1) {
        std::printf("no HIP device\n");
        return 2;
    }
    for (pkv_dtype_t dt : {PKV_BF16, PKV_F32})
        if (int rc = run_case(dt)) return rc;
    std::printf(g_failures ? "c client: %d check(s) failed\n" : "c client: all checks passed\n",
                g_failures);
    return g_failures ? 1 : 0;
}
