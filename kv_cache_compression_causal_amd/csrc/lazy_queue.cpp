// Lazy-layer priority queue (LightTransfer pages: Chinese write-up,
// "solution 2"; project page, Figure 2 caption).  After each layer of the
// prefill its (lazy ratio, layer index) enters the queue; while more than C
// layers are queued, the laziest (highest ratio) leaves and its KV cache is
// switched to the streaming version.  This bounds the prefill's KV at C full
// layers plus streaming layers at every step.
//
// Readings the pages leave open: by default the queue pushes, then pops
// while its size exceeds C (so the current layer may leave at its own step);
// the other timing the pages describe (evict the laziest queued layer before
// pushing once C are queued) is a policy flag.  Equal ratios evict the lower
// layer index first; a layer's score is the fp64 mean of its per-(batch,
// head) ratios in index order.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "lt.h"

extern "C" const char *lt_last_error(void);

namespace lt {
bool log_enabled();
void log_printf(const char *fmt, ...) __attribute__((format(printf, 1, 2)));
}  // namespace lt

namespace {

struct Entry {
    double score;
    int layer;
};

// "a ranks above b" in the max-heap: higher score, then lower layer index.
inline bool above(const Entry &a, const Entry &b) {
    return a.score > b.score || (a.score == b.score && a.layer < b.layer);
}

// KV bytes held while the prefill walks the layers (every layer the same
// sizes): n_switched layers are at their streaming size, the rest of the
// layers pushed so far at full size (plus their slice when the prefill wrote
// it).  step() gives one step's pair from the decision it made.
struct KvTally {
    int64_t full = 0, stream = 0;
    bool emit = false;
    int n_switched = 0;
    int64_t retained = 0, transient = 0;

    int64_t at_full() const { return emit ? full + stream : full; }
    // Layer `layer` was pushed under `policy` and `evicted` left (or -1).
    void step(int layer, int evicted, int policy) {
        // With eviction before the push, an earlier layer leaving at this
        // step frees its memory before the current layer's KV is counted.
        const int freed_first = policy == LT_EVICT_BEFORE_PUSH && evicted >= 0 && evicted < layer;
        const int64_t sw = n_switched + freed_first;
        transient = (layer - sw) * at_full() + sw * stream + at_full();
        if (evicted >= 0) n_switched++;
        retained = (int64_t)(layer + 1 - n_switched) * at_full() + (int64_t)n_switched * stream;
    }
};

}  // namespace

struct lt_lazy_queue {
    int L, C, next, policy;
    std::vector<Entry> heap;  // binary max-heap under above()
    bool kv_set = false;
    KvTally kv;

    // One step: layer e.layer arrives; returns the layer evicted, or -1.
    int step(const Entry &e) {
        if (policy == LT_EVICT_BEFORE_PUSH) {
            if (C == 0) return e.layer;
            const int v = (int)heap.size() == C ? pop().layer : -1;
            push(e);
            return v;
        }
        push(e);
        return (int)heap.size() > C ? pop().layer : -1;
    }

    void push(const Entry &e) {
        heap.push_back(e);
        size_t i = heap.size() - 1;
        while (i > 0) {
            size_t p = (i - 1) / 2;
            if (!above(heap[i], heap[p])) break;
            Entry t = heap[i]; heap[i] = heap[p]; heap[p] = t;
            i = p;
        }
    }
    Entry pop() {
        Entry top = heap[0];
        heap[0] = heap.back();
        heap.pop_back();
        size_t i = 0, n = heap.size();
        for (;;) {
            size_t l = 2 * i + 1, r = l + 1, best = i;
            if (l < n && above(heap[l], heap[best])) best = l;
            if (r < n && above(heap[r], heap[best])) best = r;
            if (best == i) break;
            Entry t = heap[i]; heap[i] = heap[best]; heap[best] = t;
            i = best;
        }
        return top;
    }
};

namespace {
// Shares the thread-local error text of lt_api.cpp through a tiny setter.
int qfail(int code, const char *msg);

// A layer's score: the mean of its n ratios, summed in fp64 in index order.
// Returns false if a ratio is not finite.
bool mean_of(const float *x, int n, double *out) {
    double acc = 0.0;
    for (int i = 0; i < n; ++i) {
        if (isnan(x[i]) || isinf(x[i])) return false;
        acc += (double)x[i];
    }
    *out = acc / (double)n;
    return true;
}
}  // namespace

extern "C" {

int lt_lazy_queue_create_policy(int L, int C, int policy, lt_lazy_queue **out) {
    if (out == nullptr) return qfail(LT_ERR_NULL, "out is NULL");
    if (L < 1) return qfail(LT_ERR_SHAPE, "L must be >= 1");
    if (C < 0 || C > L) return qfail(LT_ERR_VALUE, "capacity must lie in [0, L]");
    if (policy != LT_EVICT_AFTER_PUSH && policy != LT_EVICT_BEFORE_PUSH)
        return qfail(LT_ERR_VALUE, "unknown eviction policy");
    lt_lazy_queue *q = new (std::nothrow) lt_lazy_queue();
    if (q == nullptr) return qfail(LT_ERR_VALUE, "out of host memory");
    q->L = L; q->C = C; q->next = 0; q->policy = policy;
    q->heap.reserve((size_t)C + 1);
    *out = q;
    return qfail(LT_OK, "");
}

int lt_lazy_queue_create(int L, int C, lt_lazy_queue **out) {
    return lt_lazy_queue_create_policy(L, C, LT_EVICT_AFTER_PUSH, out);
}

int lt_lazy_queue_push(lt_lazy_queue *q, int layer, double score, int *evicted) {
    if (q == nullptr || evicted == nullptr) return qfail(LT_ERR_NULL, "queue/evicted is NULL");
    if (q->next >= q->L) return qfail(LT_ERR_VALUE, "all L layers have been pushed");
    if (layer != q->next) return qfail(LT_ERR_VALUE, "layers must be pushed in order");
    if (isnan(score) || isinf(score)) return qfail(LT_ERR_VALUE, "score must be finite");
    *evicted = q->step(Entry{score, layer});
    if (q->kv_set) q->kv.step(layer, *evicted, q->policy);
    q->next++;
    if (lt::log_enabled()) {
        if (q->kv_set)
            lt::log_printf("lt_lazy_queue_push(layer=%d score=%.9g) -> evicted %d, KV retained %lld transient %lld",
                           layer, score, *evicted, (long long)q->kv.retained, (long long)q->kv.transient);
        else
            lt::log_printf("lt_lazy_queue_push(layer=%d score=%.9g) -> evicted %d", layer, score, *evicted);
    }
    return qfail(LT_OK, "");
}

int lt_lazy_queue_set_kv_bytes(lt_lazy_queue *q, int64_t full_bytes, int64_t stream_bytes, int emit) {
    if (q == nullptr) return qfail(LT_ERR_NULL, "queue is NULL");
    if (full_bytes < 0 || stream_bytes < 0) return qfail(LT_ERR_VALUE, "sizes must be >= 0");
    if (q->next != 0) return qfail(LT_ERR_VALUE, "set the KV sizes before the first push");
    q->kv = KvTally{};
    q->kv.full = full_bytes;
    q->kv.stream = stream_bytes;
    q->kv.emit = emit != 0;
    q->kv_set = true;
    return qfail(LT_OK, "");
}

int lt_lazy_queue_kv_bytes(const lt_lazy_queue *q, int64_t *retained, int64_t *transient) {
    if (q == nullptr || retained == nullptr || transient == nullptr)
        return qfail(LT_ERR_NULL, "queue/retained/transient is NULL");
    if (!q->kv_set) return qfail(LT_ERR_VALUE, "KV sizes not set");
    if (q->next == 0) return qfail(LT_ERR_VALUE, "no layer pushed yet");
    *retained = q->kv.retained;
    *transient = q->kv.transient;
    return qfail(LT_OK, "");
}

int lt_kv_accounting(const int *evicted_at_step, int L, int policy, int64_t full_bytes, int64_t stream_bytes,
                     int emit, int64_t *retained, int64_t *transient) {
    if (evicted_at_step == nullptr || retained == nullptr || transient == nullptr)
        return qfail(LT_ERR_NULL, "NULL argument");
    if (L < 1) return qfail(LT_ERR_SHAPE, "L must be >= 1");
    if (policy != LT_EVICT_AFTER_PUSH && policy != LT_EVICT_BEFORE_PUSH)
        return qfail(LT_ERR_VALUE, "unknown eviction policy");
    if (full_bytes < 0 || stream_bytes < 0) return qfail(LT_ERR_VALUE, "sizes must be >= 0");
    std::vector<uint8_t> gone((size_t)L, 0);
    for (int l = 0; l < L; ++l) {
        const int e = evicted_at_step[l];
        if (e < -1 || e > l) return qfail(LT_ERR_VALUE, "evicted_at_step[l] must be -1 or a layer 0..l");
        if (e >= 0 && gone[e]++) return qfail(LT_ERR_VALUE, "a layer is evicted twice");
    }
    KvTally t;
    t.full = full_bytes;
    t.stream = stream_bytes;
    t.emit = emit != 0;
    for (int l = 0; l < L; ++l) {
        t.step(l, evicted_at_step[l], policy);
        retained[l] = t.retained;
        transient[l] = t.transient;
    }
    return qfail(LT_OK, "");
}

void lt_lazy_queue_destroy(lt_lazy_queue *q) { delete q; }

int lt_lazy_queue_push_ratios(lt_lazy_queue *q, int layer, const float *head_ratio, int n,
                              double *score, int *evicted) {
    if (q == nullptr || head_ratio == nullptr || evicted == nullptr)
        return qfail(LT_ERR_NULL, "queue/head_ratio/evicted is NULL");
    if (n < 1) return qfail(LT_ERR_SHAPE, "n must be >= 1");
    double sc;
    if (!mean_of(head_ratio, n, &sc)) return qfail(LT_ERR_VALUE, "head ratio is not finite");
    const int e = lt_lazy_queue_push(q, layer, sc, evicted);
    if (e == LT_OK && score != nullptr) *score = sc;
    return e;
}

int lt_select_lazy_layers_policy(const float *head_ratio, int L, int n, int C, int policy,
                                 double *layer_score, int *evicted_at_step, uint8_t *is_streaming) {
    if (head_ratio == nullptr || evicted_at_step == nullptr || is_streaming == nullptr)
        return qfail(LT_ERR_NULL, "NULL argument");
    if (L < 1 || n < 1) return qfail(LT_ERR_SHAPE, "L and n must be >= 1");
    if (C < 0 || C > L) return qfail(LT_ERR_VALUE, "capacity must lie in [0, L]");
    if (policy != LT_EVICT_AFTER_PUSH && policy != LT_EVICT_BEFORE_PUSH)
        return qfail(LT_ERR_VALUE, "unknown eviction policy");
    std::vector<double> score((size_t)L);
    for (int l = 0; l < L; ++l)
        if (!mean_of(head_ratio + (size_t)l * n, n, &score[l]))
            return qfail(LT_ERR_VALUE, "head ratio is not finite");
    lt_lazy_queue q;
    q.L = L; q.C = C; q.next = 0; q.policy = policy;
    q.heap.reserve((size_t)C + 1);
    for (int l = 0; l < L; ++l) is_streaming[l] = 0;
    for (int l = 0; l < L; ++l) {
        const int v = q.step(Entry{score[l], l});
        evicted_at_step[l] = v;
        if (v >= 0) is_streaming[v] = 1;
    }
    if (layer_score != nullptr)
        for (int l = 0; l < L; ++l) layer_score[l] = score[l];
    return qfail(LT_OK, "");
}

int lt_select_lazy_layers(const float *head_ratio, int L, int n, int C, double *layer_score,
                          int *evicted_at_step, uint8_t *is_streaming) {
    return lt_select_lazy_layers_policy(head_ratio, L, n, C, LT_EVICT_AFTER_PUSH, layer_score,
                                        evicted_at_step, is_streaming);
}

// Offline selection (press-release page, "LightTransfer method"): the score
// of layer l is the mean over prompts of its per-prompt score (each the
// fp64 mean of that prompt's per-(batch, head) ratios), summed in prompt
// order; the L - C highest become streaming layers, ties to the lower index.
int lt_select_offline(const float *head_ratio, int P, int L, int n, int C, double *layer_score,
                      uint8_t *is_streaming) {
    if (head_ratio == nullptr || is_streaming == nullptr) return qfail(LT_ERR_NULL, "NULL argument");
    if (P < 1 || L < 1 || n < 1) return qfail(LT_ERR_SHAPE, "P, L and n must be >= 1");
    if (C < 0 || C > L) return qfail(LT_ERR_VALUE, "capacity must lie in [0, L]");
    std::vector<double> mean((size_t)L, 0.0);
    for (int l = 0; l < L; ++l) {
        double acc = 0.0;
        for (int p = 0; p < P; ++p) {
            double sc;
            if (!mean_of(head_ratio + ((size_t)p * L + l) * n, n, &sc))
                return qfail(LT_ERR_VALUE, "head ratio is not finite");
            acc += sc;
        }
        mean[l] = acc / (double)P;
    }
    std::vector<int> order((size_t)L);
    for (int l = 0; l < L; ++l) order[l] = l;
    std::sort(order.begin(), order.end(),
              [&](int a, int b) { return above(Entry{mean[a], a}, Entry{mean[b], b}); });
    for (int l = 0; l < L; ++l) is_streaming[l] = 0;
    for (int i = 0; i < L - C; ++i) is_streaming[order[i]] = 1;
    if (layer_score != nullptr)
        for (int l = 0; l < L; ++l) layer_score[l] = mean[l];
    return qfail(LT_OK, "");
}

}  // extern "C"

namespace lt_detail {
void set_error(const char *msg);
}

namespace {
int qfail(int code, const char *msg) {
    lt_detail::set_error(msg);
    return code;
}
}  // namespace
