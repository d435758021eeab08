// Host block manager and two-phase continuous-batching scheduler (PhotonInfer
// README, "Technical details -> Paged attention" and "-> Continuous-batching
// scheduler"; "Key features -> vLLM-style continuous batching").  The rules
// are stated in include/photon_sched.h.  Pure host code: it produces the
// block tables, context lengths, slot mappings and positions that the
// decode-path kernels consume.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "photon_sched.h"
#include "status.h"

using photon::fail;
using photon::ok;

namespace {

enum State : int32_t { kWaiting = 0, kRunning = 1, kFinished = 2 };

struct Request {
    int64_t id = 0;
    int32_t prompt_len = 0;
    int32_t max_new = 0;
    int32_t num_known = 0;      // prompt + generated
    int32_t num_computed = 0;   // known tokens whose K/V are cached
    int32_t num_generated = 0;
    int32_t num_preemptions = 0;
    int32_t state = kWaiting;
    int32_t step_tokens = 0;    // new tokens in the step last scheduled
    std::vector<int32_t> blocks;
};

int32_t cdiv(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

}  // namespace

struct photon_sched {
    photon_sched_config cfg{};
    std::deque<int32_t> free_blocks;            // FIFO free list
    std::vector<Request> reqs;                  // every request ever added
    std::unordered_map<int64_t, size_t> by_id;  // request id -> index into reqs
    std::deque<size_t> waiting;                 // front is served first
    std::vector<size_t> running;                // admission order
    std::vector<size_t> scheduled;              // batch order of the last schedule()
    bool pending_update = false;
    int32_t num_finished = 0;

    void release_blocks(Request &r)
    {
        for (int32_t b : r.blocks)
            free_blocks.push_back(b);
        r.blocks.clear();
    }

    void take_blocks(Request &r, int32_t count)
    {
        for (int32_t i = 0; i < count; ++i) {
            r.blocks.push_back(free_blocks.front());
            free_blocks.pop_front();
        }
    }

    int32_t blocks_short(const Request &r, int32_t n) const
    {
        return cdiv((int64_t)r.num_computed + n, cfg.block_size) - (int32_t)r.blocks.size();
    }

    // Preempt the last running request: free its blocks, forget its cached
    // tokens and put it at the front of the waiting queue.
    size_t preempt_last()
    {
        const size_t idx = running.back();
        running.pop_back();
        Request &v = reqs[idx];
        release_blocks(v);
        v.num_computed = 0;
        v.state = kWaiting;
        ++v.num_preemptions;
        waiting.push_front(idx);
        return idx;
    }
};

extern "C" {

photon_status photon_sched_create(const photon_sched_config *config, photon_sched **out)
{
    if (!config || !out)
        return fail(PHOTON_ERR_INVALID_ARG, "config and out must not be NULL");
    const photon_sched_config &c = *config;
    if (c.num_blocks <= 0 || c.block_size <= 0 || c.max_seqs <= 0 || c.max_blocks_per_seq <= 0)
        return fail(PHOTON_ERR_INVALID_ARG,
                    "num_blocks %d, block_size %d, max_seqs %d and max_blocks_per_seq %d must be > 0",
                    c.num_blocks, c.block_size, c.max_seqs, c.max_blocks_per_seq);
    if (c.max_tokens_per_step < c.max_seqs)
        return fail(PHOTON_ERR_INVALID_ARG, "max_tokens_per_step %d must be >= max_seqs %d",
                    c.max_tokens_per_step, c.max_seqs);
    if ((int64_t)c.num_blocks * c.block_size > INT32_MAX)
        return fail(PHOTON_ERR_INVALID_ARG, "num_blocks * block_size exceeds the int32 slot range");
    photon_sched *s = new (std::nothrow) photon_sched;
    if (!s)
        return fail(PHOTON_ERR_INVALID_ARG, "out of host memory");
    s->cfg = c;
    for (int32_t b = 0; b < c.num_blocks; ++b)
        s->free_blocks.push_back(b);
    *out = s;
    return ok();
}

void photon_sched_destroy(photon_sched *sched) { delete sched; }

photon_status photon_sched_add_request(photon_sched *s, int64_t request_id, int32_t prompt_len,
                                       int32_t max_new_tokens)
{
    if (!s)
        return fail(PHOTON_ERR_INVALID_ARG, "scheduler is NULL");
    if (prompt_len < 1 || max_new_tokens < 1)
        return fail(PHOTON_ERR_INVALID_ARG, "prompt_len %d and max_new_tokens %d must be >= 1",
                    prompt_len, max_new_tokens);
    const int32_t most = cdiv((int64_t)prompt_len + max_new_tokens - 1, s->cfg.block_size);
    if (most > s->cfg.max_blocks_per_seq || most > s->cfg.num_blocks)
        return fail(PHOTON_ERR_INVALID_ARG,
                    "request %lld may need %d blocks: more than max_blocks_per_seq %d or the pool %d",
                    (long long)request_id, most, s->cfg.max_blocks_per_seq, s->cfg.num_blocks);
    if (s->by_id.count(request_id))
        return fail(PHOTON_ERR_INVALID_ARG, "request id %lld already added", (long long)request_id);
    Request r;
    r.id = request_id;
    r.prompt_len = prompt_len;
    r.max_new = max_new_tokens;
    r.num_known = prompt_len;
    s->by_id.emplace(request_id, s->reqs.size());
    s->reqs.push_back(r);
    s->waiting.push_back(s->reqs.size() - 1);
    return ok();
}

photon_status photon_sched_schedule(photon_sched *s, photon_sched_batch *batch)
{
    if (!s || !batch)
        return fail(PHOTON_ERR_INVALID_ARG, "scheduler and batch must not be NULL");
    if (s->pending_update)
        return fail(PHOTON_ERR_INVALID_ARG, "schedule() called twice without update()");
    if (!batch->request_ids || !batch->query_start || !batch->context_lens || !batch->block_tables ||
        !batch->slot_mapping || !batch->positions)
        return fail(PHOTON_ERR_INVALID_ARG, "batch arrays must not be NULL");
    const photon_sched_config &c = s->cfg;
    int32_t budget = c.max_tokens_per_step;
    int32_t preempted = 0;
    s->scheduled.clear();

    // Phase 1: every running request continues.
    for (size_t i = 0; i < s->running.size(); ++i) {
        const size_t idx = s->running[i];
        Request &r = s->reqs[idx];
        const int32_t later = (int32_t)(s->running.size() - 1 - i);
        const int32_t n = std::min(r.num_known - r.num_computed, budget - later);
        bool self_preempted = false;
        while ((int32_t)s->free_blocks.size() < s->blocks_short(r, n)) {
            const size_t victim = s->preempt_last();
            if (batch->preempted_ids)
                batch->preempted_ids[preempted] = s->reqs[victim].id;
            ++preempted;
            if (victim == idx) {
                self_preempted = true;
                break;
            }
        }
        if (self_preempted)
            break;  // it was the last running request
        s->take_blocks(r, s->blocks_short(r, n));
        r.step_tokens = n;
        budget -= n;
        s->scheduled.push_back(idx);
    }

    // Phase 2: admit waiting requests into the capacity left.
    while (!s->waiting.empty() && (int32_t)s->scheduled.size() < c.max_seqs && budget > 0) {
        const size_t idx = s->waiting.front();
        Request &r = s->reqs[idx];
        const int32_t n = std::min(r.num_known - r.num_computed, budget);
        const int32_t short_by = s->blocks_short(r, n);
        if ((int32_t)s->free_blocks.size() < short_by)
            break;
        s->waiting.pop_front();
        s->take_blocks(r, short_by);
        r.state = kRunning;
        s->running.push_back(idx);
        r.step_tokens = n;
        budget -= n;
        s->scheduled.push_back(idx);
    }

    // The path's inputs for this step.
    int32_t tok = 0;
    for (size_t b = 0; b < s->scheduled.size(); ++b) {
        const Request &r = s->reqs[s->scheduled[b]];
        batch->request_ids[b] = r.id;
        batch->query_start[b] = tok;
        for (int32_t j = 0; j < r.step_tokens; ++j, ++tok) {
            const int32_t pos = r.num_computed + j;
            batch->positions[tok] = pos;
            batch->slot_mapping[tok] = r.blocks[pos / c.block_size] * c.block_size + pos % c.block_size;
        }
        batch->context_lens[b] = r.num_computed + r.step_tokens;
        int32_t *row = batch->block_tables + b * (size_t)c.max_blocks_per_seq;
        for (int32_t k = 0; k < c.max_blocks_per_seq; ++k)
            row[k] = k < (int32_t)r.blocks.size() ? r.blocks[k] : -1;
    }
    batch->query_start[s->scheduled.size()] = tok;
    batch->num_seqs = (int32_t)s->scheduled.size();
    batch->num_tokens = tok;
    batch->num_preempted = preempted;
    s->pending_update = true;
    return ok();
}

photon_status photon_sched_update(photon_sched *s, int32_t *num_finished, int64_t *finished_ids)
{
    if (!s)
        return fail(PHOTON_ERR_INVALID_ARG, "scheduler is NULL");
    if (!s->pending_update)
        return fail(PHOTON_ERR_INVALID_ARG, "update() without a scheduled step");
    int32_t done = 0;
    for (size_t idx : s->scheduled) {
        Request &r = s->reqs[idx];
        r.num_computed += r.step_tokens;
        r.step_tokens = 0;
        if (r.num_computed == r.num_known) {
            ++r.num_generated;
            ++r.num_known;
            if (r.num_generated == r.max_new) {
                s->release_blocks(r);
                r.state = kFinished;
                s->running.erase(std::find(s->running.begin(), s->running.end(), idx));
                if (finished_ids)
                    finished_ids[done] = r.id;
                ++done;
                ++s->num_finished;
            }
        }
    }
    s->scheduled.clear();
    s->pending_update = false;
    if (num_finished)
        *num_finished = done;
    return ok();
}

photon_status photon_sched_counts(const photon_sched *s, int32_t *num_waiting, int32_t *num_running,
                                  int32_t *num_finished, int32_t *num_free_blocks)
{
    if (!s)
        return fail(PHOTON_ERR_INVALID_ARG, "scheduler is NULL");
    if (num_waiting)
        *num_waiting = (int32_t)s->waiting.size();
    if (num_running)
        *num_running = (int32_t)s->running.size();
    if (num_finished)
        *num_finished = s->num_finished;
    if (num_free_blocks)
        *num_free_blocks = (int32_t)s->free_blocks.size();
    return ok();
}

photon_status photon_sched_request(const photon_sched *s, int64_t request_id,
                                   photon_sched_request_info *info)
{
    if (!s || !info)
        return fail(PHOTON_ERR_INVALID_ARG, "scheduler and info must not be NULL");
    auto it = s->by_id.find(request_id);
    if (it == s->by_id.end())
        return fail(PHOTON_ERR_INVALID_ARG, "unknown request id %lld", (long long)request_id);
    const Request &r = s->reqs[it->second];
    info->state = r.state;
    info->num_computed = r.num_computed;
    info->num_known = r.num_known;
    info->num_generated = r.num_generated;
    info->num_blocks = (int32_t)r.blocks.size();
    info->num_preemptions = r.num_preemptions;
    return ok();
}

}  // extern "C"
