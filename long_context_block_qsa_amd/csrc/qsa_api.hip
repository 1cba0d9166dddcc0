// qsa_api.hip -- the C ABI declared in include/qsa.h: host-side validation,
// workspace layout and launch orchestration. Nothing is enqueued before every
// argument has been checked; no device memory is allocated here.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <vector>

#pragma GCC visibility push(default)
#include "qsa.h"
#pragma GCC visibility pop
#include "qsa_device.h"
#include "qsa_launch.h"

// ------------------------------------------------------------ kernel trace
namespace qsa {
namespace {
struct Trace {
    bool open = false;
    bool pending = false;
    bool failed = false;
    int cap = 0, n = 0;
    std::vector<hipEvent_t> ev;   // 2 per kernel
    std::vector<int> kind;
};
thread_local Trace g_trace;
}  // namespace

void trace_before(int kind, hipStream_t st) {
    Trace &t = g_trace;
    t.pending = false;
    if (!t.open || t.n >= t.cap) return;
    if (hipEventRecord(t.ev[2 * t.n], st) != hipSuccess) { t.failed = true; return; }
    t.kind[t.n] = kind;
    t.pending = true;
}

hipError_t trace_after(hipStream_t st, hipError_t launch_status) {
    Trace &t = g_trace;
    if (t.pending) {
        t.pending = false;
        if (hipEventRecord(t.ev[2 * t.n + 1], st) != hipSuccess) t.failed = true;
        else ++t.n;
    }
    return launch_status;
}
}  // namespace qsa

namespace {

using qsa::SeqInfo;

constexpr size_t kAlign = 256;
constexpr int kMaxGridY = 65535;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Host mirrors of the device bookkeeping formulas.
int64_t h_slots_before(int64_t t) {
    int64_t m = t / 4, r = t % 4;
    return 2 * m * (m - 1) + m * (r + 1);
}
int64_t h_first_scored_pos(int64_t L, int64_t nq, int64_t topk) {
    return std::max(L - nq, 4 * topk + 3);
}

// Prefill-shaped calls select in passes: a pass is a run of whole score tiles (with the
// rows they cover and the unscored rows before them) whose score keys fit kKeyBudget
// slots. Two key buffers alternate: one launch selects the rows of pass p from one
// buffer while it scores pass p + 1 into the other, so the workspace does not grow
// with the square of the context and no pass ends with its own tail.
// slots (uint32 keys) per buffer: 256 MiB (2^25 took 47.5 ms of score + select for a
// 262,144-token prefill, 2^26 39.9 ms, 2^27 41.2 ms: more rows per launch, until the two
// buffers outgrow the Infinity Cache)
constexpr int64_t kKeyBudget = int64_t(1) << 26;

struct Pass {
    int64_t tile_lo = 0, tile_hi = 0;   // score tiles
    int64_t row_lo = 0, row_hi = 0;     // query rows selected after the pass is scored
    int64_t slot_lo = 0, slot_hi = 0;   // score slots (keys[s - slot_lo])
    int64_t max_blocks = 0;             // most blocks a row of the pass sees
    int64_t chunk = 0;                  // blocks per scoring workgroup
    bool long_rows = false;             // max_blocks > SEL_LONG_KEYS: the long-row kernel
};

struct Plan {
    int batch = 0;
    int topk = 0;
    float scale = 0.f;
    int64_t tq = 0, tk = 0;
    int64_t n_tiles = 0;        // score tiles (4 query rows each)
    int64_t n_slots = 0;        // fp32 score slots
    int64_t max_score_blocks = 0;
    int64_t max_len = 0;        // longest sequence
    int64_t max_cmp_full = 0;   // most complete blocks in a sequence
    int64_t max_cmp_incr = 0;   // most blocks holding a query token
    int local_ch = 0;           // > 0: decode path, blocks per chunk
    int max_chunks = 0;         // chunks of the longest scored row (decode path)
    int nsplit = 1;             // attention key splits per row
    int64_t n_dense = 0;        // query rows with at most topk visible blocks
    int64_t n_dense_tiles = 0;  // their tiles of DN_ROWS rows (per sequence)
    size_t off_ctl = 0, off_tab = 0, off_sel = 0, off_union = 0, off_cand = 0,
           off_part = 0;
    size_t ws_bytes = 0;
    bool use_dec = false;       // few rows: row/tile tables travel as kernel arguments
    bool fuse_compress = false; // decode: scoring workgroups compress the new blocks
    bool merge_launch = false;  // decode: some tile's rows are merged by their own launch
    qsa::DecodeTables dec;
    std::vector<Pass> passes;   // prefill-shaped calls
    int64_t pass_slots = 0;     // largest pass (slots of the keys buffer)
};

// Cuts the score tiles of a prefill-shaped call into passes of at most `budget` slots
// (a single tile larger than the budget gets a pass of its own). Tiles, rows and
// slots are numbered as on the device: sequences in order, a sequence's tiles cover
// its rows at t >= first scored position, 4 rows each.
qsa_status build_passes(const int32_t *cq, const int32_t *ck, int batch, int topk,
                        int64_t budget, Plan *p) {
    Pass cur;
    int64_t tile = 0, slot = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t L = (int64_t)ck[b + 1] - ck[b], nq = (int64_t)cq[b + 1] - cq[b];
        const int64_t ts = h_first_scored_pos(L, nq, topk);
        for (int64_t t0 = ts; t0 < L; t0 += 4, ++tile) {
            const int64_t nr = std::min<int64_t>(4, L - t0);
            const int64_t row0 = cq[b] + (t0 - (L - nq));
            const int64_t ns = h_slots_before(t0 + nr) - h_slots_before(t0);
            if (cur.slot_hi > cur.slot_lo && cur.slot_hi - cur.slot_lo + ns > budget) {
                cur.tile_hi = tile;
                cur.row_hi = row0;
                p->passes.push_back(cur);
                cur = Pass();
                cur.tile_lo = tile;
                cur.row_lo = row0;
                cur.slot_lo = cur.slot_hi = slot;
            }
            slot += ns;
            cur.slot_hi = slot;
            cur.max_blocks = std::max(cur.max_blocks, (t0 + nr) / qsa::BS);
        }
    }
    cur.tile_hi = tile;
    cur.row_hi = cq[batch];
    p->passes.push_back(cur);
    for (Pass &ps : p->passes) {
        p->pass_slots = std::max(p->pass_slots, ps.slot_hi - ps.slot_lo);
        const int64_t nt = ps.tile_hi - ps.tile_lo;
        if (nt <= 0) continue;
        // enough workgroups to fill the chip when the pass has few tiles (the long-row
        // kernel scores 4 tiles per workgroup)
        ps.long_rows = ps.max_blocks > qsa::SEL_LONG_KEYS;
        const int64_t ngr = ps.long_rows ? (nt + 3) / 4 : nt;
        int64_t gy = std::max<int64_t>(1, (2048 + ngr - 1) / ngr);
        gy = std::min<int64_t>(gy, std::max<int64_t>(1, ps.max_blocks / 256));
        int64_t chunk = (ps.max_blocks + gy - 1) / gy;
        chunk = (chunk + 63) / 64 * 64;
        ps.chunk = chunk;
        if ((ps.max_blocks + chunk - 1) / chunk > kMaxGridY || nt > INT32_MAX)
            return QSA_ERR_UNSUPPORTED;
    }
    return QSA_OK;
}

// Row and tile tables of a call with at most DEC_MAX query rows and score tiles.
void build_decode_tables(const int32_t *cq, const int32_t *ck, int batch, int topk,
                         qsa::DecodeTables *d) {
    int64_t blk = 0, slots = 0, tiles = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t L = (int64_t)ck[b + 1] - ck[b], nq = (int64_t)cq[b + 1] - cq[b];
        const int64_t ts = h_first_scored_pos(L, nq, topk);
        for (int64_t r = cq[b]; r < cq[b + 1]; ++r) {
            const int64_t t = L - nq + (r - cq[b]);
            qsa::DecRow &x = d->row[r];
            x.k0 = ck[b];
            x.t = (int32_t)t;
            x.blk0 = (int32_t)blk;
            x.tile = -1;
            x.slot = t >= ts ? slots + h_slots_before(t) - h_slots_before(ts) : 0;
        }
        if (ts < L) {
            const int64_t nt = (L - ts + 3) / 4;
            for (int64_t i = 0; i < nt; ++i) {
                qsa::DecTile &y = d->tile[tiles + i];
                y.row0 = (int32_t)(cq[b] + (ts + 4 * i - (L - nq)));
                y.nrows = (int32_t)std::min<int64_t>(4, L - (ts + 4 * i));
                y.new_lo = (int32_t)((L - nq) / qsa::BS);
                y.new_hi = (int32_t)(L / qsa::BS);
                for (int32_t rr = 0; rr < y.nrows; ++rr) d->row[y.row0 + rr].tile = (int32_t)(tiles + i);
            }
            tiles += nt;
            slots += h_slots_before(L) - h_slots_before(ts);
        }
        blk += L / qsa::BS;
    }
}

qsa_status check_dims(const qsa_dims *d) {
    if (!d) return QSA_ERR_NULL;
    if (d->n_q_heads != qsa::HQ || d->n_kv_heads != qsa::HKV || d->head_dim != qsa::HD ||
        d->n_idx_heads != qsa::HI || d->idx_dim != qsa::DI || d->block_size != qsa::BS)
        return QSA_ERR_UNSUPPORTED;
    if (d->topk_blocks < 1 || d->topk_blocks > qsa::KMAX) return QSA_ERR_SHAPE;
    if (!isfinite(d->softmax_scale)) return QSA_ERR_SHAPE;
    return QSA_OK;
}

// Validates the sequence description and fills the plan. need_q: cu_q is used.
qsa_status make_plan(const qsa_dims *d, const qsa_seqs *s, bool need_q, Plan *p) {
    qsa_status st = check_dims(d);
    if (st != QSA_OK) return st;
    if (!s) return QSA_ERR_NULL;
    if (s->batch < 0) return QSA_ERR_SHAPE;
    if (s->batch > kMaxGridY) return QSA_ERR_UNSUPPORTED;
    if (!s->cu_k_host || (need_q && !s->cu_q_host)) return QSA_ERR_NULL;
    if (s->batch > 0 && (!s->cu_k_dev || (need_q && !s->cu_q_dev))) return QSA_ERR_NULL;
    const int32_t *ck = s->cu_k_host, *cq = need_q ? s->cu_q_host : nullptr;
    if (ck[0] != 0 || (cq && cq[0] != 0)) return QSA_ERR_SHAPE;
    p->batch = s->batch;
    p->topk = d->topk_blocks;
    p->scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)qsa::HD);
    for (int b = 0; b < s->batch; ++b) {
        const int64_t L = (int64_t)ck[b + 1] - ck[b];
        if (L < 0) return QSA_ERR_SHAPE;
        int64_t nq = 0;
        if (cq) {
            nq = (int64_t)cq[b + 1] - cq[b];
            if (nq < 0 || nq > L) return QSA_ERR_SHAPE;
        }
        p->max_len = std::max(p->max_len, L);
        p->max_cmp_full = std::max(p->max_cmp_full, L / qsa::BS);
        if (nq > 0)
            p->max_cmp_incr = std::max(p->max_cmp_incr, L / qsa::BS - (L - nq) / qsa::BS);
        const int64_t ts = h_first_scored_pos(L, nq, p->topk);
        if (cq) {
            const int64_t nd = std::max<int64_t>(0, std::min(ts, L) - (L - nq));
            p->n_dense += nd;
            p->n_dense_tiles += (nd + qsa::DN_ROWS - 1) / qsa::DN_ROWS;
        }
        if (cq && ts < L) {
            p->n_tiles += (L - ts + 3) / 4;
            p->n_slots += h_slots_before(L) - h_slots_before(ts);
            p->max_score_blocks = std::max(p->max_score_blocks, L / qsa::BS);
        }
    }
    p->tk = ck[s->batch];
    p->tq = cq ? cq[s->batch] : 0;
    if (p->n_tiles > INT32_MAX) return QSA_ERR_UNSUPPORTED;

    p->use_dec = cq && p->tq <= qsa::DEC_MAX && p->n_tiles <= qsa::DEC_MAX;
    if (p->use_dec) {
        build_decode_tables(cq, ck, p->batch, p->topk, &p->dec);
        // new blocks can be compressed by the scoring kernel when every sequence that
        // has one also has a score tile (its last tile covers all of its blocks)
        p->fuse_compress = true;
        for (int b = 0; b < p->batch; ++b) {
            const int64_t L = (int64_t)ck[b + 1] - ck[b], nq = (int64_t)cq[b + 1] - cq[b];
            const bool has_new = nq > 0 && L / qsa::BS > (L - nq) / qsa::BS;
            if (has_new && h_first_scored_pos(L, nq, p->topk) >= L) p->fuse_compress = false;
        }
    }
    // decode path: few score tiles over long rows -> chunked scoring with local
    // candidates; the chunk shrinks until the longest row's full chunks offer twice the
    // budget in candidates (with exactly the budget every candidate would be kept, which
    // the merge cannot tell from a chunk hiding better blocks: the row would always take
    // the exact path)
    constexpr int kKP = 32;
    // (rows with too few chunks for candidates are selected from their full key row)
    if (p->use_dec && p->n_tiles > 0) {
        int ch = 1024;
        while (ch > 64 && (p->max_score_blocks / ch) * kKP < 2 * (int64_t)p->topk) ch /= 2;
        p->local_ch = ch;
        p->max_chunks = (int)((p->max_score_blocks + ch - 1) / ch);
        if (p->max_chunks > kMaxGridY) return QSA_ERR_UNSUPPORTED;
        // the merge launch serves tiles whose chunks fit one merge
        for (int64_t i = 0; i < p->n_tiles && !p->merge_launch; ++i) {
            const qsa::DecTile &tl = p->dec.tile[i];
            const int64_t nv_max = ((int64_t)p->dec.row[tl.row0].t + tl.nrows) / qsa::BS;
            p->merge_launch = (nv_max + ch - 1) / ch <= qsa::MERGE_CHUNKS_WIDE;
        }
    }
    // prefill-shaped calls: passes of whole score tiles under the key budget
    if (cq && !p->use_dec) {
        const qsa_status ps = build_passes(cq, ck, p->batch, p->topk, kKeyBudget, p);
        if (ps != QSA_OK) return ps;
    }
    // attention splits: aim at ~1024 waves when rows are few
    if (p->tq > 0) {
        int64_t ns = (1024 + 2 * p->tq - 1) / (2 * p->tq);
        p->nsplit = (int)std::min<int64_t>(64, std::max<int64_t>(1, ns));
        // a workgroup's 4 waves are consecutive splits of one (row, KV head) when nsplit
        // is a multiple of 4: they merge their partials through LDS first (4x fewer
        // partials for the combine). Decode rows merged inside the attention need at
        // least whole rows per workgroup (nsplit even).
        if (p->nsplit >= 4) p->nsplit = (p->nsplit + 3) / 4 * 4;
        else if (p->local_ch > 0 && p->nsplit > 1) p->nsplit += p->nsplit & 1;
    }
    // workspace: [control block][seq table][selection][scores | attention partials]
    const size_t ctl_b = (size_t)qsa::CTL_WORDS * sizeof(uint32_t);
    const size_t tab_b = align_up((size_t)std::max(p->batch, 1) * sizeof(SeqInfo));
    const size_t sel_b = align_up((size_t)p->tq * (size_t)p->topk * sizeof(int32_t));
    // prefill: two key buffers when there is more than one pass
    const size_t score_b = p->use_dec
        ? align_up((size_t)p->n_slots * sizeof(uint32_t))
        : align_up((size_t)p->pass_slots * sizeof(uint32_t)) * (p->passes.size() > 1 ? 2 : 1);
    const size_t cand_b = p->local_ch > 0
        ? align_up((size_t)p->tq * p->max_chunks * kKP * 2 * sizeof(uint32_t)) : 0;
    const size_t part_b = p->nsplit > 1
        ? align_up((size_t)p->tq * p->nsplit * qsa::HQ * (qsa::HD + 4) * sizeof(float)) : 0;
    p->off_ctl = 0;
    p->off_tab = ctl_b;
    p->off_sel = ctl_b + tab_b;
    p->off_union = ctl_b + tab_b + sel_b;  // scores (+ candidates) while selecting, then partials
    p->off_cand = p->off_union + score_b;
    // decode (chunk candidates): the attention reads the candidates while it writes its
    // partials, so they get their own space; otherwise the partials reuse the scores'
    p->off_part = p->local_ch > 0 ? p->off_cand + cand_b : p->off_union;
    p->ws_bytes = p->local_ch > 0 ? p->off_part + part_b
                                  : p->off_union + std::max(score_b + cand_b, part_b);
    return QSA_OK;
}

qsa_status check_ws(const Plan &p, void *ws, size_t ws_bytes) {
    if (!ws) return QSA_ERR_NULL;
    if (((uintptr_t)ws % kAlign) != 0) return QSA_ERR_WORKSPACE;
    if (ws_bytes < p.ws_bytes) return QSA_ERR_WORKSPACE;
    return QSA_OK;
}

qsa_status device_status(hipError_t e) { return e == hipSuccess ? QSA_OK : QSA_ERR_DEVICE; }
qsa_status device_status(qsa_status s) { return s; }

// A second stream per host thread and device (default priority, created on first use and
// kept), with events reused by this thread's calls: prefill forwards attend the rows of
// each selection pass on it while the caller's stream scores and selects the next passes.
// Events are only recorded and waited on, so the fork and join also record into a graph
// the caller's stream is capturing.
struct SideStreams {
    std::vector<hipStream_t> stream;            // per device
    std::vector<std::vector<hipEvent_t>> ev;    // per device
};
thread_local SideStreams tl_side;

qsa_status side_stream(size_t n_events, hipStream_t *side, hipEvent_t **ev) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return QSA_ERR_DEVICE;
    if ((size_t)dev >= tl_side.stream.size()) {
        tl_side.stream.resize(dev + 1, nullptr);
        tl_side.ev.resize(dev + 1);
    }
    if (!tl_side.stream[dev] &&
        hipStreamCreateWithFlags(&tl_side.stream[dev], hipStreamNonBlocking) != hipSuccess) {
        tl_side.stream[dev] = nullptr;
        return QSA_ERR_DEVICE;
    }
    std::vector<hipEvent_t> &e = tl_side.ev[dev];
    while (e.size() < n_events) {
        hipEvent_t x;
        if (hipEventCreateWithFlags(&x, hipEventDisableTiming) != hipSuccess) return QSA_ERR_DEVICE;
        e.push_back(x);
    }
    *side = tl_side.stream[dev];
    *ev = e.data();
    return QSA_OK;
}

#define QSA_TRY(expr)                                  \
    do {                                               \
        qsa_status _s = device_status(expr);           \
        if (_s != QSA_OK) return _s;                   \
    } while (0)

template <typename T>
T *ws_at(void *ws, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }

// merge_in_attend: the decode rows merged after scoring are merged by the attention
// launch that follows (forward), not by a merge launch here.
// The forward attends the rows in the dense regime with the dense-tile kernel (bf16 K/V,
// prefill-shaped calls without attention splits); with no scored row at all, that kernel
// also writes the selections and no select launch is needed.
bool dense_tile_path(const Plan &p, bool fp8) {
    return !fp8 && !p.use_dec && p.nsplit == 1 && p.n_dense_tiles > 0;
}
bool sel_by_dense_tiles(const Plan &p, bool fp8) { return dense_tile_path(p, fp8) && p.n_tiles == 0; }

// after_pass (prefill, not null): called once the launch that selects pass i's rows has
// been enqueued, with i.
template <class AfterPass = std::nullptr_t>
qsa_status run_select(const Plan &p, const qsa_seqs *s, const qsa_bf16 *q_idx, const float *w,
                      const qsa_bf16 *k_idx, qsa_bf16 *k_blk, int32_t *sel, void *ws,
                      hipStream_t st, bool merge_in_attend = false, bool sel_by_dense = false,
                      AfterPass after_pass = nullptr) {
    SeqInfo *tab = ws_at<SeqInfo>(ws, p.off_tab);
    uint32_t *keys = ws_at<uint32_t>(ws, p.off_union);
    uint32_t *cand_key = nullptr;
    int32_t *cand_idx = nullptr;
    if (p.local_ch > 0) {
        cand_key = ws_at<uint32_t>(ws, p.off_cand);
        cand_idx = reinterpret_cast<int32_t *>(cand_key + (size_t)p.tq * p.max_chunks * 32);
        // scoring selects the scored rows itself; a select launch remains only for rows
        // within the budget
        QSA_TRY(qsa::launch_score_local(p.dec, p.n_tiles, p.topk, q_idx, w, k_idx, k_blk, keys,
                                        cand_key, cand_idx, p.local_ch, p.max_chunks, sel,
                                        ws_at<uint32_t>(ws, p.off_ctl), st));
        // rows whose chunks fit one merge are merged one workgroup per row
        if (p.merge_launch && !merge_in_attend)
            QSA_TRY(qsa::launch_merge_dec(p.dec, p.tq, p.topk, q_idx, w, k_blk, keys, cand_key,
                                          cand_idx, p.local_ch, p.max_chunks, sel, st));
        if (p.n_dense > 0)
            QSA_TRY(qsa::launch_select(tab, &p.dec, p.batch, p.topk, keys, 0, cand_key,
                                       cand_idx, p.local_ch, p.max_chunks, sel, 0, p.tq, 1,
                                       st));
        return QSA_OK;
    }
    if (p.use_dec) {   // decode-shaped call without scored rows
        QSA_TRY(qsa::launch_select(tab, &p.dec, p.batch, p.topk, keys, 0, nullptr, nullptr, 0,
                                   0, sel, 0, p.tq, 0, st));
        return QSA_OK;
    }
    if (sel_by_dense) return QSA_OK;
    // prefill: launch i scores pass i into buffer i % 2 and selects the rows of pass
    // i - 1 from buffer (i - 1) % 2
    uint32_t *buf[2] = {keys, keys + align_up((size_t)p.pass_slots * sizeof(uint32_t)) / 4};
    const size_t np = p.passes.size();
    for (size_t i = 0; i <= np; ++i) {
        const Pass *sc = i < np ? &p.passes[i] : nullptr;
        const Pass *se = i > 0 ? &p.passes[i - 1] : nullptr;
        QSA_TRY(qsa::launch_score_select(
            tab, p.batch, p.topk, q_idx, w, k_blk, buf[i % 2], sc ? sc->tile_lo : 0,
            sc ? sc->tile_hi - sc->tile_lo : 0, sc ? sc->slot_lo : 0, sc ? sc->max_blocks : 0,
            sc ? sc->chunk : 1, buf[(i + 1) % 2], se ? se->slot_lo : 0, sel,
            se ? se->row_lo : 0, se ? se->row_hi - se->row_lo : 0,
            (sc && sc->long_rows) || (se && se->long_rows), st));
        if constexpr (!std::is_same<AfterPass, std::nullptr_t>::value)
            if (i > 0) QSA_TRY(after_pass(i - 1));
    }
    (void)s;
    return QSA_OK;
}

// dense_tiles: the selection is the library's own (a forward step), so rows with at
// most topk visible blocks keep them all and are attended by the dense-regime kernel;
// sel_out (not null) is where that kernel writes their selections.
qsa_status run_attend(const Plan &p, const qsa_bf16 *q, const qsa_bf16 *k, const qsa_bf16 *v,
                      const qsa::Fp8Kv *fp8, const int32_t *sel, float *out, float *lse,
                      void *ws, hipStream_t st, const qsa::AttnMerge *merge = nullptr,
                      bool dense_tiles = false, int32_t *sel_out = nullptr) {
    SeqInfo *tab = ws_at<SeqInfo>(ws, p.off_tab);
    float *part = ws_at<float>(ws, p.off_part);
    const bool dense = dense_tiles && dense_tile_path(p, fp8 != nullptr);
    if (dense)
        QSA_TRY(qsa::launch_attend_dense(tab, p.batch, p.topk, p.scale, q, k, v, out, lse,
                                         sel_out, p.n_dense_tiles, st));
    if (!dense || p.n_dense < p.tq)
        QSA_TRY(qsa::launch_attend(tab, p.use_dec ? &p.dec : nullptr, p.batch, p.topk, p.scale,
                                   q, k, v, fp8, sel, out, lse, part, p.nsplit, p.tq, merge,
                                   dense, st));
    return QSA_OK;
}

// The attention addresses a sequence's K and V with 32-bit byte offsets.
constexpr int64_t kMaxAttendLen = int64_t(1) << 22;

qsa_status attend_common(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                         const qsa_bf16 *k, const qsa_bf16 *v, const qsa::Fp8Kv *fp8,
                         const int32_t *sel, float *out, float *lse, void *ws, size_t ws_bytes,
                         void *stream) {
    Plan p;
    qsa_status st = make_plan(dims, seqs, true, &p);
    if (st != QSA_OK) return st;
    if (p.max_len > kMaxAttendLen) return QSA_ERR_UNSUPPORTED;
    if (p.tq == 0) return QSA_OK;
    if (!q || !sel || !out) return QSA_ERR_NULL;
    if (fp8 ? (!fp8->k8 || !fp8->v8 || !fp8->k_scale || !fp8->v_scale) : (!k || !v))
        return QSA_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || !aligned16(sel) ||
        (fp8 ? (!aligned16(fp8->k8) || !aligned16(fp8->v8) || !aligned16(fp8->k_scale) ||
                !aligned16(fp8->v_scale))
             : (!aligned16(k) || !aligned16(v))))
        return QSA_ERR_SHAPE;
    if ((st = check_ws(p, ws, ws_bytes)) != QSA_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    if (!p.use_dec)
        QSA_TRY(qsa::launch_prep(seqs->cu_q_dev, seqs->cu_k_dev, p.batch, p.topk,
                                 ws_at<SeqInfo>(ws, p.off_tab), hs));
    return run_attend(p, q, k, v, fp8, sel, out, lse, ws, hs);
}

// overlap: prefill calls of several selection passes may attend each pass's rows on the
// thread's side stream (not for callers that cannot allocate: creating it allocates).
qsa_status forward_common(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                          const qsa_bf16 *k, const qsa_bf16 *v, const qsa::Fp8Kv *fp8,
                          const qsa_bf16 *q_idx, const float *w, const qsa_bf16 *k_idx,
                          qsa_bf16 *k_blk, int32_t *sel, float *out, float *lse, void *ws,
                          size_t ws_bytes, void *stream, bool overlap = true) {
    Plan p;
    qsa_status st = make_plan(dims, seqs, true, &p);
    if (st != QSA_OK) return st;
    if (p.max_len > kMaxAttendLen) return QSA_ERR_UNSUPPORTED;
    if (p.tq == 0) return QSA_OK;
    if (!q || !out) return QSA_ERR_NULL;
    if (fp8 ? (!fp8->k8 || !fp8->v8 || !fp8->k_scale || !fp8->v_scale) : (!k || !v))
        return QSA_ERR_NULL;
    if (p.n_tiles > 0 && (!q_idx || !w)) return QSA_ERR_NULL;
    if ((p.n_tiles > 0 || (k_idx && p.max_cmp_incr > 0)) && !k_blk) return QSA_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || (q_idx && !aligned16(q_idx)) ||
        (w && !aligned16(w)) || (k_idx && !aligned16(k_idx)) || (k_blk && !aligned16(k_blk)) ||
        (sel && !aligned16(sel)) ||
        (fp8 ? (!aligned16(fp8->k8) || !aligned16(fp8->v8) || !aligned16(fp8->k_scale) ||
                !aligned16(fp8->v_scale))
             : (!aligned16(k) || !aligned16(v))))
        return QSA_ERR_SHAPE;
    if ((st = check_ws(p, ws, ws_bytes)) != QSA_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    int32_t *sel_use = sel ? sel : ws_at<int32_t>(ws, p.off_sel);
    SeqInfo *tab = p.use_dec ? nullptr : ws_at<SeqInfo>(ws, p.off_tab);
    const bool fused = p.use_dec && p.fuse_compress && k_idx && p.n_tiles > 0;
    if (k_idx && p.max_cmp_incr > 0 && !fused)   // compress the new blocks (and build the table)
        QSA_TRY(qsa::launch_compress(seqs->cu_q_dev, seqs->cu_k_dev, p.batch, p.max_cmp_incr,
                                     k_idx, k_blk, 1, tab, p.topk, hs));
    else if (!p.use_dec)
        QSA_TRY(qsa::launch_prep(seqs->cu_q_dev, seqs->cu_k_dev, p.batch, p.topk, tab, hs));
    // decode rows merged after scoring: the attention workgroups of a row merge its
    // candidates themselves (no merge launch, no selection round trip through memory)
    const bool merge_in_attend = p.use_dec && p.local_ch > 0 && p.merge_launch;
    const bool sel_by_dense = sel_by_dense_tiles(p, fp8 != nullptr);
    // prefill in several selection passes: the rows of pass i are attended on the side
    // stream as soon as the launch that selects them has run, while the caller's stream
    // scores and selects the later passes (the attention reads only the selections of its
    // own rows; the key buffers the later launches reuse are the selection's alone). Only
    // where it pays: the FP8 attention (bound by its instruction issue as much as by its
    // gathers) and prefills with long-row passes (rows of more than SEL_LONG_KEYS blocks);
    // the bf16 attention of shorter rows is bound by the L2 requests of its gathers, and
    // sharing the L2 with the selection passes made the whole step slower.
    const bool long_passes = std::any_of(p.passes.begin(), p.passes.end(),
                                         [](const Pass &ps) { return ps.long_rows; });
    if (overlap && !p.use_dec && p.nsplit == 1 && p.passes.size() > 1 && !sel_by_dense &&
        (fp8 != nullptr || long_passes)) {
        hipStream_t side;
        hipEvent_t *ev;
        const size_t np = p.passes.size();
        if ((st = side_stream(np + 1, &side, &ev)) != QSA_OK) return st;
        const bool dense = dense_tile_path(p, fp8 != nullptr);
        auto after_pass = [&](size_t i) -> qsa_status {
            const Pass &ps = p.passes[i];
            QSA_TRY(hipEventRecord(ev[i], hs));
            QSA_TRY(hipStreamWaitEvent(side, ev[i], 0));
            QSA_TRY(qsa::launch_attend(tab, nullptr, p.batch, p.topk, p.scale, q, k, v, fp8,
                                       sel_use, out, lse, ws_at<float>(ws, p.off_part), 1,
                                       ps.row_hi - ps.row_lo, nullptr, dense, side, ps.row_lo));
            return QSA_OK;
        };
        st = run_select(p, seqs, q_idx, w, nullptr, k_blk, sel_use, ws, hs, false, false,
                        after_pass);
        // the dense-regime rows on the caller's stream meanwhile; then it waits for the side
        // stream's attention (also after an error above, so nothing is left unjoined)
        if (st == QSA_OK && dense)
            st = device_status(qsa::launch_attend_dense(tab, p.batch, p.topk, p.scale, q, k, v,
                                                        out, lse, nullptr, p.n_dense_tiles, hs));
        const qsa_status jst = device_status(hipEventRecord(ev[np], side));
        const qsa_status wst = jst == QSA_OK ? device_status(hipStreamWaitEvent(hs, ev[np], 0)) : jst;
        return st != QSA_OK ? st : wst;
    }
    if ((st = run_select(p, seqs, q_idx, w, fused ? k_idx : nullptr, k_blk, sel_use, ws, hs,
                         merge_in_attend, sel_by_dense)) != QSA_OK)
        return st;
    qsa::AttnMerge m = {};
    if (merge_in_attend) {
        m.q_idx = q_idx; m.w = w; m.k_blk = k_blk;
        m.keys = ws_at<uint32_t>(ws, p.off_union);
        m.cand_key = ws_at<uint32_t>(ws, p.off_cand);
        m.cand_idx = reinterpret_cast<int32_t *>(m.cand_key + (size_t)p.tq * p.max_chunks * 32);
        m.ch = p.local_ch; m.max_chunks = p.max_chunks;
        m.sel = sel_use;
    }
    return run_attend(p, q, k, v, fp8, sel_use, out, lse, ws, hs, merge_in_attend ? &m : nullptr,
                      true, sel_by_dense ? sel_use : nullptr);
}

// Attention backward: per-sequence table, D, nsel, list offsets, block totals, count
// matrices and block -> rows lists after the control block.
struct BwdPlan {
    Plan p;
    int64_t n_chunks = 0, nkb_total = 0, mat_entries = 0, max_entries = 0;
    size_t off_seq = 0, off_delta = 0, off_nsel = 0, off_off = 0, off_tot = 0, off_mat = 0,
           off_list = 0, ws_bytes = 0;
};

qsa_status make_bwd_plan(const qsa_dims *d, const qsa_seqs *s, BwdPlan *bp) {
    qsa_status st = make_plan(d, s, true, &bp->p);
    if (st != QSA_OK) return st;
    const int32_t *ck = s->cu_k_host, *cq = s->cu_q_host;
    for (int b = 0; b < s->batch; ++b) {
        const int64_t L = (int64_t)ck[b + 1] - ck[b], nq = (int64_t)cq[b + 1] - cq[b];
        const int64_t nkb = (L + qsa::BS - 1) / qsa::BS, nch = (nq + qsa::BWD_CH - 1) / qsa::BWD_CH;
        bp->nkb_total += nkb;
        bp->n_chunks += nch;
        bp->mat_entries += nkb * nch;
    }
    // every row attends at most topk selected blocks and its raw tail: list positions,
    // block offsets and counts stay within int32
    bp->max_entries = bp->p.tq * (int64_t)(bp->p.topk + 1);
    if (bp->max_entries > INT32_MAX || bp->nkb_total >= INT32_MAX ||
        bp->n_chunks > INT32_MAX)
        return QSA_ERR_UNSUPPORTED;
    const size_t ctl_b = (size_t)qsa::CTL_WORDS * sizeof(uint32_t);
    size_t o = ctl_b;
    bp->off_seq = o;   o += align_up((size_t)std::max(s->batch, 1) * sizeof(qsa::BwdSeq));
    bp->off_delta = o; o += align_up((size_t)bp->p.tq * qsa::HQ * sizeof(float));
    bp->off_nsel = o;  o += align_up((size_t)bp->p.tq * sizeof(int32_t));
    bp->off_off = o;   o += align_up((size_t)(bp->nkb_total + 1) * sizeof(int32_t));
    bp->off_tot = o;   o += align_up((size_t)bp->nkb_total * sizeof(int32_t));
    bp->off_mat = o;   o += align_up((size_t)bp->mat_entries * sizeof(int32_t));
    bp->off_list = o;  o += align_up((size_t)bp->max_entries * sizeof(int32_t));
    bp->ws_bytes = o;
    return QSA_OK;
}

// ------------------------------------------------- scratch of qsa_forward_noalloc
// The workspace of the no-allocation entry point: one array per GPU, part of the
// library's code object (it exists on every device the library is loaded on, until
// the process ends). In host code `scratch` only names the symbol: its device address
// comes from hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __attribute__((aligned(256))) uint8_t scratch[QSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // per device, guarded by g_scratch_mu

// The current device's scratch address. On the first call for a device its control
// block is cleared by a kernel on `st` (the array is zero when the code object is
// loaded; the clear makes that explicit, and in a captured graph it is a kernel node).
qsa_status noalloc_scratch(hipStream_t st, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QSA_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return QSA_ERR_DEVICE;
        if (qsa::launch_zero_words(static_cast<uint32_t *>(ptr), qsa::CTL_WORDS, st) !=
            hipSuccess)
            return QSA_ERR_DEVICE;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return QSA_OK;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int32_t qsa_abi_version(void) { return QSA_ABI_VERSION; }

const char *qsa_status_string(int32_t s) {
    switch (s) {
    case QSA_OK: return "QSA_OK";
    case QSA_ERR_NULL: return "QSA_ERR_NULL: a required pointer is NULL";
    case QSA_ERR_SHAPE: return "QSA_ERR_SHAPE: invalid sequence offsets, budget or alignment";
    case QSA_ERR_UNSUPPORTED: return "QSA_ERR_UNSUPPORTED: dims or sizes outside the supported set";
    case QSA_ERR_WORKSPACE: return "QSA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case QSA_ERR_DEVICE: return "QSA_ERR_DEVICE: a kernel launch failed";
    }
    return "unknown qsa_status";
}

qsa_status qsa_workspace_size(const qsa_dims *dims, const qsa_seqs *seqs, size_t *bytes) {
    if (!bytes) return QSA_ERR_NULL;
    Plan p;
    qsa_status st = make_plan(dims, seqs, true, &p);
    if (st != QSA_OK) return st;
    *bytes = p.ws_bytes;
    return QSA_OK;
}

qsa_status qsa_compress(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *k_idx,
                        qsa_bf16 *k_blk, void *stream) {
    Plan p;
    qsa_status st = make_plan(dims, seqs, false, &p);
    if (st != QSA_OK) return st;
    if (p.max_cmp_full == 0) return QSA_OK;
    if (!k_idx || !k_blk) return QSA_ERR_NULL;
    if (!aligned16(k_idx) || !aligned16(k_blk)) return QSA_ERR_SHAPE;
    QSA_TRY(qsa::launch_compress(nullptr, seqs->cu_k_dev, p.batch, p.max_cmp_full, k_idx, k_blk,
                                 0, nullptr, p.topk, (hipStream_t)stream));
    return QSA_OK;
}

qsa_status qsa_select(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q_idx,
                      const float *w, const qsa_bf16 *k_blk, int32_t *sel, void *ws,
                      size_t ws_bytes, void *stream) {
    Plan p;
    qsa_status st = make_plan(dims, seqs, true, &p);
    if (st != QSA_OK) return st;
    if (p.tq == 0) return QSA_OK;
    if (!sel) return QSA_ERR_NULL;
    if (p.n_tiles > 0 && (!q_idx || !w || !k_blk)) return QSA_ERR_NULL;
    if ((q_idx && !aligned16(q_idx)) || (k_blk && !aligned16(k_blk)) ||
        (w && !aligned16(w)) || !aligned16(sel))
        return QSA_ERR_SHAPE;
    if ((st = check_ws(p, ws, ws_bytes)) != QSA_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    if (!p.use_dec)
        QSA_TRY(qsa::launch_prep(seqs->cu_q_dev, seqs->cu_k_dev, p.batch, p.topk,
                                 ws_at<SeqInfo>(ws, p.off_tab), hs));
    return run_select(p, seqs, q_idx, w, nullptr, const_cast<qsa_bf16 *>(k_blk), sel, ws, hs);
}

qsa_status qsa_score(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q_idx,
                     const float *w, const qsa_bf16 *k_blk, const int64_t *rows, int64_t n_rows,
                     float *scores, int64_t ld, void *stream) {
    Plan p;
    qsa_status st = make_plan(dims, seqs, true, &p);
    if (st != QSA_OK) return st;
    if (n_rows < 0 || n_rows > INT32_MAX || ld < 0) return QSA_ERR_SHAPE;
    if (n_rows == 0) return QSA_OK;
    if (p.tq == 0 || ld < p.max_cmp_full) return QSA_ERR_SHAPE;
    if (ld == 0) return QSA_OK;
    if (!rows || !scores || !q_idx || !w || (p.max_cmp_full > 0 && !k_blk)) return QSA_ERR_NULL;
    if (!aligned16(q_idx) || !aligned16(w) || (k_blk && !aligned16(k_blk)))
        return QSA_ERR_SHAPE;
    QSA_TRY(qsa::launch_score_rows(seqs->cu_q_dev, seqs->cu_k_dev, p.batch, rows, n_rows, q_idx,
                                   w, k_blk, scores, ld, (hipStream_t)stream));
    return QSA_OK;
}

qsa_status qsa_attend(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                      const qsa_bf16 *k, const qsa_bf16 *v, const int32_t *sel, float *out,
                      float *lse, void *ws, size_t ws_bytes, void *stream) {
    return attend_common(dims, seqs, q, k, v, nullptr, sel, out, lse, ws, ws_bytes, stream);
}

qsa_status qsa_forward(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                       const qsa_bf16 *k, const qsa_bf16 *v, const qsa_bf16 *q_idx,
                       const float *w, const qsa_bf16 *k_idx, qsa_bf16 *k_blk, int32_t *sel,
                       float *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
    return forward_common(dims, seqs, q, k, v, nullptr, q_idx, w, k_idx, k_blk, sel, out, lse,
                          ws, ws_bytes, stream);
}

qsa_status qsa_forward_noalloc(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                               const qsa_bf16 *k, const qsa_bf16 *v, const qsa_bf16 *q_idx,
                               const float *w, const qsa_bf16 *k_idx, qsa_bf16 *k_blk,
                               int32_t *sel, float *out, float *lse, void *stream) {
    // the call's workspace must fit the scratch; checked before any device call
    Plan p;
    qsa_status st = make_plan(dims, seqs, true, &p);
    if (st != QSA_OK) return st;
    if (p.max_len > kMaxAttendLen) return QSA_ERR_UNSUPPORTED;
    if (p.tq == 0) return QSA_OK;
    if (p.ws_bytes > (size_t)QSA_NOALLOC_SCRATCH_BYTES) return QSA_ERR_WORKSPACE;
    if (!q || !out) return QSA_ERR_NULL;
    void *ws = nullptr;
    if ((st = noalloc_scratch((hipStream_t)stream, &ws)) != QSA_OK) return st;
    return forward_common(dims, seqs, q, k, v, nullptr, q_idx, w, k_idx, k_blk, sel, out, lse,
                          ws, (size_t)QSA_NOALLOC_SCRATCH_BYTES, stream, false);
}

qsa_status qsa_quantize_kv(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *k,
                           const qsa_bf16 *v, uint8_t *k8, uint8_t *v8, float *k_scale,
                           float *v_scale, void *stream) {
    Plan p;
    qsa_status st = make_plan(dims, seqs, false, &p);
    if (st != QSA_OK) return st;
    if (p.tk == 0) return QSA_OK;
    if (!k || !v || !k8 || !v8 || !k_scale || !v_scale) return QSA_ERR_NULL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k8) || !aligned16(v8) ||
        !aligned16(k_scale) || !aligned16(v_scale))
        return QSA_ERR_SHAPE;
    QSA_TRY(qsa::launch_quantize_kv(k, v, k8, v8, k_scale, v_scale, p.tk * qsa::HKV,
                                    (hipStream_t)stream));
    return QSA_OK;
}

qsa_status qsa_attend_fp8(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                          const uint8_t *k8, const uint8_t *v8, const float *k_scale,
                          const float *v_scale, const int32_t *sel, float *out, float *lse,
                          void *ws, size_t ws_bytes, void *stream) {
    const qsa::Fp8Kv f = {k8, v8, k_scale, v_scale};
    return attend_common(dims, seqs, q, nullptr, nullptr, &f, sel, out, lse, ws, ws_bytes,
                         stream);
}

qsa_status qsa_forward_fp8(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                           const uint8_t *k8, const uint8_t *v8, const float *k_scale,
                           const float *v_scale, const qsa_bf16 *q_idx, const float *w,
                           const qsa_bf16 *k_idx, qsa_bf16 *k_blk, int32_t *sel, float *out,
                           float *lse, void *ws, size_t ws_bytes, void *stream) {
    const qsa::Fp8Kv f = {k8, v8, k_scale, v_scale};
    return forward_common(dims, seqs, q, nullptr, nullptr, &f, q_idx, w, k_idx, k_blk, sel,
                          out, lse, ws, ws_bytes, stream);
}

qsa_status qsa_backward_workspace_size(const qsa_dims *dims, const qsa_seqs *seqs,
                                       size_t *bytes) {
    if (!bytes) return QSA_ERR_NULL;
    BwdPlan bp;
    qsa_status st = make_bwd_plan(dims, seqs, &bp);
    if (st != QSA_OK) return st;
    *bytes = bp.ws_bytes;
    return QSA_OK;
}

qsa_status qsa_attend_backward(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                               const qsa_bf16 *k, const qsa_bf16 *v, const int32_t *sel,
                               const float *out, const float *lse, const qsa_bf16 *dout,
                               float *dq, float *dk, float *dv, void *ws, size_t ws_bytes,
                               void *stream) {
    BwdPlan bp;
    qsa_status st = make_bwd_plan(dims, seqs, &bp);
    if (st != QSA_OK) return st;
    const Plan &p = bp.p;
    if (p.tq == 0 && p.tk == 0) return QSA_OK;
    if (p.tk > 0 && (!k || !v || !dk || !dv)) return QSA_ERR_NULL;
    if (p.tq > 0 && (!q || !sel || !out || !lse || !dout || !dq)) return QSA_ERR_NULL;
    if ((q && !aligned16(q)) || (k && !aligned16(k)) || (v && !aligned16(v)) ||
        (sel && !aligned16(sel)) || (out && !aligned16(out)) || (lse && !aligned16(lse)) ||
        (dout && !aligned16(dout)) || (dq && !aligned16(dq)) || (dk && !aligned16(dk)) ||
        (dv && !aligned16(dv)))
        return QSA_ERR_SHAPE;
    if (!ws) return QSA_ERR_NULL;
    if (((uintptr_t)ws % kAlign) != 0 || ws_bytes < bp.ws_bytes) return QSA_ERR_WORKSPACE;
    qsa::BwdBuffers b;
    b.seq = ws_at<qsa::BwdSeq>(ws, bp.off_seq);
    b.delta = ws_at<float>(ws, bp.off_delta);
    b.nsel = ws_at<int32_t>(ws, bp.off_nsel);
    b.off = ws_at<int32_t>(ws, bp.off_off);
    b.tot = ws_at<int32_t>(ws, bp.off_tot);
    b.mat = ws_at<int32_t>(ws, bp.off_mat);
    b.list = ws_at<int32_t>(ws, bp.off_list);
    // dQ on the thread's side stream, concurrently with dK/dV on the caller's
    hipStream_t side;
    hipEvent_t *ev;
    if ((st = side_stream(2, &side, &ev)) != QSA_OK) return st;
    QSA_TRY(qsa::launch_backward(seqs->cu_q_dev, seqs->cu_k_dev, seqs->cu_q_host,
                                 seqs->cu_k_host, p.batch, p.topk, p.scale, p.tq,
                                 bp.n_chunks, bp.nkb_total, q, k, v, sel, out, lse, dout, dq,
                                 dk, dv, b, (hipStream_t)stream, side, ev[0], ev[1]));
    return QSA_OK;
}

qsa_status qsa_trace_begin(int32_t max_kernels) {
    qsa::Trace &t = qsa::g_trace;
    if (t.open || max_kernels < 1 || max_kernels > (1 << 20)) return QSA_ERR_SHAPE;
    t.ev.assign(2 * (size_t)max_kernels, nullptr);
    t.kind.assign((size_t)max_kernels, -1);
    for (auto &e : t.ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            for (auto &x : t.ev)
                if (x) (void)hipEventDestroy(x);   // best effort on the error path
            t.ev.clear();
            return QSA_ERR_DEVICE;
        }
    }
    t.cap = max_kernels;
    t.n = 0;
    t.failed = false;
    t.pending = false;
    t.open = true;
    return QSA_OK;
}

int32_t qsa_trace_end(int32_t max_out, int32_t *kind_out, float *ms_out) {
    qsa::Trace &t = qsa::g_trace;
    if (!t.open) return -1;
    int32_t n = t.n;
    bool ok = !t.failed;
    for (int i = 0; i < n && ok; ++i) {
        float ms = 0.f;
        if (hipEventSynchronize(t.ev[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess) {
            ok = false;
            break;
        }
        if (i < max_out) {
            if (kind_out) kind_out[i] = t.kind[i];
            if (ms_out) ms_out[i] = ms;
        }
    }
    for (auto &e : t.ev) (void)hipEventDestroy(e);   // nothing to report once the times are read
    t.ev.clear();
    t.kind.clear();
    t.open = false;
    t.n = 0;
    return ok ? n : -1;
}

const char *qsa_kernel_name(int32_t kind) {
    static const char *names[] = {"prep",     "compress",    "score",    "select",
                                  "attend",   "combine",     "bwd_prep", "bwd_rows",
                                  "bwd_count", "bwd_colscan", "bwd_scan", "bwd_fill",
                                  "bwd_dq",   "bwd_dkv",     "score_select", "attend_dense"};
    return (kind >= 0 && kind < 16) ? names[kind] : "unknown";
}

}  // extern "C"
#pragma GCC visibility pop
