// plan_drive.cpp -- runs the library's host-side planning and argument validation
// under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU. Every call here
// either sizes a workspace or is rejected before any device call is made; the device
// pointers handed in are never dereferenced on the host (they are aligned stand-ins).
//
// Built by tests/test_sanitizers.py with the host sanitizers only (hipcc -Xarch_host).
// Exit status 0 and no sanitizer report mean the host code is clean on these inputs.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "qsa.h"

namespace {

int g_fail = 0;

#define EXPECT(cond)                                                                 \
    do {                                                                             \
        if (!(cond)) {                                                               \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                                \
        }                                                                            \
    } while (0)

qsa_dims model_dims(int topk) {
    qsa_dims d;
    d.n_q_heads = 24; d.n_kv_heads = 2; d.head_dim = 128;
    d.n_idx_heads = 4; d.idx_dim = 64; d.block_size = 4;
    d.topk_blocks = topk; d.softmax_scale = 0.f;
    return d;
}

// Offsets of a batch given lengths and query counts (the queries are each sequence's
// last tokens).
struct Batch {
    std::vector<int32_t> cu_q, cu_k;
    Batch(const std::vector<int64_t> &lens, const std::vector<int64_t> &q_lens) {
        cu_q.assign(1, 0);
        cu_k.assign(1, 0);
        for (size_t i = 0; i < lens.size(); ++i) {
            cu_k.push_back((int32_t)(cu_k.back() + lens[i]));
            cu_q.push_back((int32_t)(cu_q.back() + q_lens[i]));
        }
    }
    qsa_seqs seqs() const {
        qsa_seqs s;
        s.batch = (int32_t)(cu_k.size() - 1);
        s.cu_q_host = cu_q.data();
        s.cu_k_host = cu_k.data();
        // stand-ins for device copies: only checked for NULL on the host
        s.cu_q_dev = reinterpret_cast<const int32_t *>(uintptr_t(0x10000));
        s.cu_k_dev = reinterpret_cast<const int32_t *>(uintptr_t(0x20000));
        return s;
    }
};

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {   // xorshift64*
    g_rng ^= g_rng >> 12;
    g_rng ^= g_rng << 25;
    g_rng ^= g_rng >> 27;
    return g_rng * 2685821657736338717ull;
}
int64_t uniform(int64_t lo, int64_t hi) {   // [lo, hi]
    return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1));
}

// Sizes the forward and backward workspaces of a valid batch.
void size_valid(const Batch &b, int topk) {
    const qsa_dims d = model_dims(topk);
    const qsa_seqs s = b.seqs();
    size_t fw = 0, bw = 0;
    EXPECT(qsa_workspace_size(&d, &s, &fw) == QSA_OK);
    EXPECT(qsa_backward_workspace_size(&d, &s, &bw) == QSA_OK);
    if (s.cu_q_host[s.batch] > 0) EXPECT(fw > 0);
}

void* fake(uintptr_t a) { return reinterpret_cast<void *>(a); }

}  // namespace

int main() {
    // ---- constants and names
    EXPECT(qsa_abi_version() == QSA_ABI_VERSION);
    for (int st = -2; st <= 7; ++st) EXPECT(qsa_status_string(st) != nullptr);
    for (int k = -3; k <= 20; ++k) EXPECT(qsa_kernel_name(k) != nullptr);

    // ---- workspace sizes of the shapes the library serves
    size_valid(Batch({}, {}), 512);
    size_valid(Batch({0}, {0}), 512);
    size_valid(Batch({1}, {1}), 1);
    size_valid(Batch({7, 1, 2, 3, 0, 64}, {7, 1, 2, 3, 0, 64}), 4);
    size_valid(Batch({1024}, {1024}), 512);
    size_valid(Batch({16384}, {16384}), 512);
    size_valid(Batch({65535, 40001, 8190, 3}, {65535, 40001, 8190, 3}), 512);
    size_valid(Batch({262144}, {262144}), 512);
    size_valid(Batch({1048576}, {1048576}), 512);   // many key passes
    size_valid(Batch({32768}, {1}), 512);
    size_valid(Batch(std::vector<int64_t>(16, 262144), std::vector<int64_t>(16, 1)), 512);
    size_valid(Batch(std::vector<int64_t>(16, 262144), std::vector<int64_t>(16, 4)), 512);
    size_valid(Batch(std::vector<int64_t>(4, 1048576), std::vector<int64_t>(4, 1)), 512);
    size_valid(Batch(std::vector<int64_t>(64, 5000), std::vector<int64_t>(64, 1)), 512);
    size_valid(Batch(std::vector<int64_t>(65, 5000), std::vector<int64_t>(65, 1)), 512);
    size_valid(Batch({4099, 2052, 2051, 2050}, {1, 2052, 2051, 7}), 512);
    // random ragged batches: lengths 0 .. 20000, any number of query tokens, any budget
    for (int it = 0; it < 300; ++it) {
        const int nb = (int)uniform(1, 40);
        std::vector<int64_t> lens, ql;
        for (int i = 0; i < nb; ++i) {
            const int64_t L = uniform(0, 1) ? uniform(0, 20000) : uniform(0, 40);
            lens.push_back(L);
            const int64_t kind = uniform(0, 3);
            ql.push_back(kind == 0 ? L : kind == 1 ? std::min<int64_t>(L, 1) : uniform(0, L));
        }
        size_valid(Batch(lens, ql), (int)uniform(1, 512));
    }

    // ---- invalid descriptions are rejected
    {
        qsa_dims d = model_dims(512);
        Batch b({100, 50}, {10, 5});
        qsa_seqs s = b.seqs();
        size_t ws = 0;
        EXPECT(qsa_workspace_size(nullptr, &s, &ws) == QSA_ERR_NULL);
        EXPECT(qsa_workspace_size(&d, nullptr, &ws) == QSA_ERR_NULL);
        EXPECT(qsa_workspace_size(&d, &s, nullptr) == QSA_ERR_NULL);
        qsa_dims bad = d; bad.topk_blocks = 0;
        EXPECT(qsa_workspace_size(&bad, &s, &ws) == QSA_ERR_SHAPE);
        bad = d; bad.topk_blocks = 513;
        EXPECT(qsa_workspace_size(&bad, &s, &ws) == QSA_ERR_SHAPE);
        bad = d; bad.n_q_heads = 32;
        EXPECT(qsa_workspace_size(&bad, &s, &ws) == QSA_ERR_UNSUPPORTED);
        bad = d; bad.block_size = 8;
        EXPECT(qsa_workspace_size(&bad, &s, &ws) == QSA_ERR_UNSUPPORTED);
        bad = d; bad.softmax_scale = 0.f / 0.f;
        EXPECT(qsa_workspace_size(&bad, &s, &ws) == QSA_ERR_SHAPE);
        qsa_seqs t = s; t.batch = -1;
        EXPECT(qsa_workspace_size(&d, &t, &ws) == QSA_ERR_SHAPE);
        t = s; t.cu_k_host = nullptr;
        EXPECT(qsa_workspace_size(&d, &t, &ws) == QSA_ERR_NULL);
        t = s; t.cu_q_dev = nullptr;
        EXPECT(qsa_workspace_size(&d, &t, &ws) == QSA_ERR_NULL);
        std::vector<int32_t> ck = {1, 100, 150}, cq = {0, 10, 15};
        t = s; t.cu_k_host = ck.data(); t.cu_q_host = cq.data();
        EXPECT(qsa_workspace_size(&d, &t, &ws) == QSA_ERR_SHAPE);      // cu_k[0] != 0
        ck = {0, 100, 90};
        EXPECT(qsa_workspace_size(&d, &t, &ws) == QSA_ERR_SHAPE);      // negative length
        ck = {0, 100, 150}; cq = {0, 120, 125};
        EXPECT(qsa_workspace_size(&d, &t, &ws) == QSA_ERR_SHAPE);      // more queries than keys
        std::vector<int32_t> big_k(70001), big_q(70001);
        for (int i = 0; i < 70001; ++i) { big_k[i] = i; big_q[i] = i; }
        t.batch = 70000; t.cu_k_host = big_k.data(); t.cu_q_host = big_q.data();
        EXPECT(qsa_workspace_size(&d, &t, &ws) == QSA_ERR_UNSUPPORTED);  // batch > grid limit
    }

    // ---- entry points reject missing, misaligned or short buffers before any device call
    {
        const qsa_dims d = model_dims(64);
        Batch b({3000, 70}, {3000, 2});
        const qsa_seqs s = b.seqs();
        size_t need = 0;
        EXPECT(qsa_workspace_size(&d, &s, &need) == QSA_OK);
        void *q = fake(0x100000), *k = fake(0x200000), *v = fake(0x300000);
        void *qi = fake(0x400000), *w = fake(0x500000), *ki = fake(0x600000);
        void *kb = fake(0x700000), *sel = fake(0x800000), *out = fake(0x900000);
        void *lse = fake(0xA00000), *ws = fake(0x1000000);
        auto fwd = [&](void *q_, void *k_, void *ws_, size_t bytes) {
            return qsa_forward(&d, &s, (const qsa_bf16 *)q_, (const qsa_bf16 *)k_,
                               (const qsa_bf16 *)v, (const qsa_bf16 *)qi, (const float *)w,
                               (const qsa_bf16 *)ki, (qsa_bf16 *)kb, (int32_t *)sel,
                               (float *)out, (float *)lse, ws_, bytes, nullptr);
        };
        EXPECT(fwd(nullptr, k, ws, need) == QSA_ERR_NULL);
        EXPECT(fwd(q, nullptr, ws, need) == QSA_ERR_NULL);
        EXPECT(fwd(fake(0x100008), k, ws, need) == QSA_ERR_SHAPE);      // q misaligned
        EXPECT(fwd(q, k, nullptr, need) == QSA_ERR_NULL);
        EXPECT(fwd(q, k, fake(0x1000010), need) == QSA_ERR_WORKSPACE);  // ws not 256-aligned
        EXPECT(fwd(q, k, ws, need - 1) == QSA_ERR_WORKSPACE);
        EXPECT(qsa_select(&d, &s, (const qsa_bf16 *)qi, (const float *)w,
                          (const qsa_bf16 *)kb, nullptr, ws, need, nullptr) == QSA_ERR_NULL);
        EXPECT(qsa_select(&d, &s, (const qsa_bf16 *)qi, (const float *)w,
                          (const qsa_bf16 *)kb, (int32_t *)sel, ws, 0, nullptr) ==
               QSA_ERR_WORKSPACE);
        EXPECT(qsa_attend(&d, &s, (const qsa_bf16 *)q, (const qsa_bf16 *)k,
                          (const qsa_bf16 *)v, nullptr, (float *)out, (float *)lse, ws, need,
                          nullptr) == QSA_ERR_NULL);
        EXPECT(qsa_compress(&d, &s, nullptr, (qsa_bf16 *)kb, nullptr) == QSA_ERR_NULL);
        EXPECT(qsa_score(&d, &s, (const qsa_bf16 *)qi, (const float *)w, (const qsa_bf16 *)kb,
                         (const int64_t *)sel, -1, (float *)out, 1000, nullptr) ==
               QSA_ERR_SHAPE);
        EXPECT(qsa_score(&d, &s, (const qsa_bf16 *)qi, (const float *)w, (const qsa_bf16 *)kb,
                         (const int64_t *)sel, 4, (float *)out, 10, nullptr) == QSA_ERR_SHAPE);
        EXPECT(qsa_quantize_kv(&d, &s, (const qsa_bf16 *)k, nullptr, (uint8_t *)kb,
                               (uint8_t *)sel, (float *)out, (float *)lse, nullptr) ==
               QSA_ERR_NULL);
        size_t bneed = 0;
        EXPECT(qsa_backward_workspace_size(&d, &s, &bneed) == QSA_OK);
        EXPECT(qsa_attend_backward(&d, &s, (const qsa_bf16 *)q, (const qsa_bf16 *)k,
                                   (const qsa_bf16 *)v, (const int32_t *)sel,
                                   (const float *)out, (const float *)lse, nullptr,
                                   (float *)qi, (float *)ki, (float *)kb, ws, bneed,
                                   nullptr) == QSA_ERR_NULL);
        EXPECT(qsa_attend_backward(&d, &s, (const qsa_bf16 *)q, (const qsa_bf16 *)k,
                                   (const qsa_bf16 *)v, (const int32_t *)sel,
                                   (const float *)out, (const float *)lse,
                                   (const qsa_bf16 *)w, (float *)qi, (float *)ki,
                                   (float *)kb, ws, bneed - 1, nullptr) == QSA_ERR_WORKSPACE);
        // a call whose workspace exceeds the no-allocation scratch is refused up front
        Batch big({65535, 40001}, {65535, 40001});
        const qsa_seqs sb = big.seqs();
        const qsa_dims d5 = model_dims(512);
        EXPECT(qsa_forward_noalloc(&d5, &sb, (const qsa_bf16 *)q, (const qsa_bf16 *)k,
                                   (const qsa_bf16 *)v, (const qsa_bf16 *)qi, (const float *)w,
                                   (const qsa_bf16 *)ki, (qsa_bf16 *)kb, (int32_t *)sel,
                                   (float *)out, (float *)lse, nullptr) == QSA_ERR_WORKSPACE);
        // attention calls address a sequence with 32-bit byte offsets
        Batch huge({(int64_t(1) << 22) + 4}, {1});
        const qsa_seqs sh = huge.seqs();
        EXPECT(qsa_attend(&d5, &sh, (const qsa_bf16 *)q, (const qsa_bf16 *)k,
                          (const qsa_bf16 *)v, (const int32_t *)sel, (float *)out,
                          (float *)lse, ws, (size_t)1 << 40, nullptr) == QSA_ERR_UNSUPPORTED);
    }

    // ---- kernel timing: end without begin, bad sizes
    EXPECT(qsa_trace_end(0, nullptr, nullptr) == -1);
    EXPECT(qsa_trace_begin(0) == QSA_ERR_SHAPE);
    EXPECT(qsa_trace_begin((1 << 20) + 1) == QSA_ERR_SHAPE);

    if (g_fail) {
        fprintf(stderr, "%d expectation(s) failed\n", g_fail);
        return 1;
    }
    printf("plan_drive: ok\n");
    return 0;
}
