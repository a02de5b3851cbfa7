// Host-side block manager and step scheduler of libpa.so: the input side of
// the attention path.  It owns no device memory; each step it produces the
// arrays the kernels take (slot_mapping, block tables, sequence and query
// lengths, copy-on-write pairs).
//
// What it follows:
//  - "AI Infra入门干货总结：大模型是如何高效推理的", section "连续批处理
//    (Continuous Batching)": a request tracks the tokens it has computed and the
//    tokens it holds (prompt + output); each step schedules the difference,
//    bounded by the running-request limit, the per-step token budget, the
//    model's maximum length and the free KV blocks.  Section "Paged Attention":
//    slot = block_table[pos / block_size] * block_size + pos % block_size.
//    Appendix 4 (preemption): when a running request cannot get blocks, the
//    lowest-priority running request frees all its blocks, its computed count
//    goes back to 0 and it returns to the front of the waiting queue; a
//    waiting request that cannot get blocks is left waiting for a later step.
//  - The inference field notes' prefix-caching entry: full blocks are hashed
//    and reused, so a shared prompt is not computed twice; their chapter on
//    batching and memory names copy-on-write for shared blocks.
//
// Policy readings (the pages leave them open): running requests keep their
// arrival order and the newest is preempted first; a prefix hit never covers
// a request's last prompt token (its block is then recomputed, so no step
// writes into a block another request shares); blocks freed by a request go
// to the back of the free list last block first, and allocation takes the
// front (least recently freed first), evicting its prefix-cache entry.
#include <stdint.h>

#include <algorithm>
#include <deque>
#include <memory>
#include <unordered_map>
#include <vector>

#include "host_status.h"

namespace {

constexpr int32_t kBlockSize = 16;
constexpr int32_t kNone = -1;

// 64-bit hash of one full block given its predecessor's hash: splitmix64
// finalisation over a running combination.  Hits are verified against the
// stored tokens and parent hash, so a collision costs only a miss.
uint64_t mix(uint64_t x) {
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}
uint64_t block_hash(uint64_t parent, const int32_t* tokens) {
    uint64_t h = mix(parent ^ 0x5A5A5A5A5A5A5A5Aull);
    for (int i = 0; i < kBlockSize; ++i) h = mix(h ^ (uint32_t)tokens[i]);
    return h;
}

struct Block {
    int32_t ref = 0;
    int32_t prev = kNone, next = kNone;   // free-list links
    bool in_free = true;
    bool cached = false;                  // registered in the prefix map under `hash`
    uint64_t hash = 0, parent = 0;
    int32_t tokens[kBlockSize] = {};
};

struct Request {
    int64_t id = 0;
    std::vector<int32_t> tokens;          // prompt, then output tokens
    int32_t num_computed = 0;
    std::vector<int32_t> blocks;          // physical block of logical block i
    std::vector<uint64_t> hashes;         // hash chain of the leading full, computed blocks
    bool running = false;
};

struct Scheduled {
    Request* req;
    int32_t start, count;                 // positions start .. start+count-1 are computed this step
};

}  // namespace

struct pa_kvm {
    int32_t num_blocks, max_num_seqs, max_batched_tokens, max_model_len, max_blocks_per_req;
    bool prefix_caching;
    std::vector<Block> blocks;
    int32_t free_head = kNone, free_tail = kNone, num_free = 0;
    std::unordered_map<uint64_t, int32_t> cache;
    std::unordered_map<int64_t, std::unique_ptr<Request>> reqs;
    std::deque<Request*> waiting;
    std::vector<Request*> running;
    // the last step's outputs (valid until the next pa_kvm_schedule)
    std::vector<Scheduled> sched;
    bool committed = true;
    // Copy sources of the current step: one freed before the step is
    // committed waits here rather than on the free list, so that no later
    // allocation of the same step makes it a copy destination while its own
    // copy is pending (the pairs of one copy launch run concurrently).
    std::vector<char> is_src;
    std::vector<int32_t> parked;
    std::vector<int64_t> out_ids, out_preempted, out_slots, out_copies;
    std::vector<int32_t> out_qlen, out_cu, out_seqlen, out_table, out_tokens, out_pos;

    // ---- free list
    void push_back(int32_t b) {
        Block& x = blocks[b];
        x.prev = free_tail;
        x.next = kNone;
        if (free_tail != kNone) blocks[free_tail].next = b; else free_head = b;
        free_tail = b;
        x.in_free = true;
        ++num_free;
    }
    void unlink(int32_t b) {
        Block& x = blocks[b];
        if (x.prev != kNone) blocks[x.prev].next = x.next; else free_head = x.next;
        if (x.next != kNone) blocks[x.next].prev = x.prev; else free_tail = x.prev;
        x.prev = x.next = kNone;
        x.in_free = false;
        --num_free;
    }
    int32_t take() {                       // a fresh block, its cached content evicted
        if (free_head == kNone) return kNone;
        const int32_t b = free_head;
        unlink(b);
        Block& x = blocks[b];
        if (x.cached) {
            auto it = cache.find(x.hash);
            if (it != cache.end() && it->second == b) cache.erase(it);
            x.cached = false;
        }
        x.ref = 1;
        return b;
    }
    void release(int32_t b) {
        if (--blocks[b].ref > 0) return;
        if (is_src[b]) parked.push_back(b);
        else push_back(b);
    }
    void end_step() {
        for (size_t i = 0; i < out_copies.size(); i += 2) is_src[out_copies[i]] = 0;
        for (int32_t b : parked)
            if (blocks[b].ref == 0) push_back(b);
        parked.clear();
    }
    void free_blocks(Request* r) {
        for (auto it = r->blocks.rbegin(); it != r->blocks.rend(); ++it) release(*it);
        r->blocks.clear();
        r->hashes.clear();
    }

    // ---- prefix cache
    // Leading full prompt blocks of r found in the cache, never its last token.
    void acquire_prefix(Request* r) {
        if (!prefix_caching) return;
        const int32_t n = (int32_t)r->tokens.size();
        const int32_t full = (n - 1) / kBlockSize;          // blocks that end before the last token
        uint64_t parent = 0;
        for (int32_t i = 0; i < full; ++i) {
            const int32_t* t = r->tokens.data() + (size_t)i * kBlockSize;
            const uint64_t h = block_hash(parent, t);
            auto it = cache.find(h);
            if (it == cache.end()) break;
            Block& x = blocks[it->second];
            if (x.parent != parent || !std::equal(t, t + kBlockSize, x.tokens)) break;
            if (x.in_free) unlink(it->second);
            ++x.ref;
            r->blocks.push_back(it->second);
            r->hashes.push_back(h);
            parent = h;
        }
        r->num_computed = (int32_t)r->blocks.size() * kBlockSize;
    }
    // Hash and register the full blocks r has computed and not yet registered.
    void register_full(Request* r) {
        if (!prefix_caching) return;
        const int32_t full = std::min(r->num_computed / kBlockSize, (int32_t)r->blocks.size());
        while ((int32_t)r->hashes.size() < full) {
            const int32_t i = (int32_t)r->hashes.size();
            const uint64_t parent = i ? r->hashes[i - 1] : 0;
            const int32_t* t = r->tokens.data() + (size_t)i * kBlockSize;
            const uint64_t h = block_hash(parent, t);
            r->hashes.push_back(h);
            const int32_t b = r->blocks[i];
            Block& x = blocks[b];
            if (!x.cached && cache.find(h) == cache.end()) {
                x.cached = true;
                x.hash = h;
                x.parent = parent;
                std::copy(t, t + kBlockSize, x.tokens);
                cache.emplace(h, b);
            }
        }
    }

    // ---- blocks for a step: positions [start, start + count) of r
    // Returns false (having changed nothing) when the free list is too short.
    bool reserve(Request* r, int32_t start, int32_t count, std::vector<int64_t>& copies) {
        const int32_t have = (int32_t)r->blocks.size();
        const int32_t need_total = (start + count + kBlockSize - 1) / kBlockSize;
        const int32_t first = start / kBlockSize;
        // copy-on-write: the block the step starts writing in is shared
        const bool cow = first < have && blocks[r->blocks[first]].ref > 1;
        const int32_t fresh = std::max(need_total - have, 0) + (cow ? 1 : 0);
        if (fresh > num_free) return false;
        if (cow) {
            const int32_t old = r->blocks[first];
            const int32_t b = take();
            is_src[old] = 1;
            copies.push_back(old);
            copies.push_back(b);
            release(old);
            r->blocks[first] = b;
            if ((int32_t)r->hashes.size() > first) r->hashes.resize(first);
        }
        while ((int32_t)r->blocks.size() < need_total) r->blocks.push_back(take());
        return true;
    }
    void preempt(Request* r) {
        free_blocks(r);
        r->num_computed = 0;
        r->running = false;
        waiting.push_front(r);
        out_preempted.push_back(r->id);
    }
};

extern "C" {

pa_kvm* pa_kvm_create(int32_t num_blocks, int32_t max_num_seqs, int32_t max_num_batched_tokens,
                      int32_t max_model_len, int32_t enable_prefix_caching) {
    if (num_blocks <= 0 || max_num_seqs <= 0 || max_num_batched_tokens <= 0 || max_model_len <= 0) {
        pa::report(PA_ERR_INVALID_ARG, "pa_kvm_create: sizes must be positive");
        return nullptr;
    }
    auto m = new pa_kvm();
    m->num_blocks = num_blocks;
    m->max_num_seqs = max_num_seqs;
    m->max_batched_tokens = max_num_batched_tokens;
    m->max_model_len = max_model_len;
    m->max_blocks_per_req = (max_model_len + kBlockSize - 1) / kBlockSize;
    m->prefix_caching = enable_prefix_caching != 0;
    m->blocks.resize(num_blocks);
    m->is_src.assign(num_blocks, 0);
    for (int32_t b = 0; b < num_blocks; ++b) m->push_back(b);
    pa::report_ok();
    return m;
}

void pa_kvm_destroy(pa_kvm* m) { delete m; }

pa_status pa_kvm_add_request(pa_kvm* m, int64_t id, const int32_t* prompt, int32_t prompt_len) {
    if (!m || (!prompt && prompt_len > 0)) return pa::report(PA_ERR_INVALID_ARG, "null pointer");
    if (prompt_len <= 0 || prompt_len > m->max_model_len)
        return pa::report(PA_ERR_INVALID_ARG, "prompt of %d tokens (1 .. max_model_len %d)", prompt_len,
                          m->max_model_len);
    if (m->reqs.count(id)) return pa::report(PA_ERR_INVALID_ARG, "request %lld exists", (long long)id);
    auto r = std::make_unique<Request>();
    r->id = id;
    r->tokens.assign(prompt, prompt + prompt_len);
    m->waiting.push_back(r.get());
    m->reqs.emplace(id, std::move(r));
    return pa::report_ok();
}

pa_status pa_kvm_fork(pa_kvm* m, int64_t parent, int64_t child) {
    if (!m) return pa::report(PA_ERR_INVALID_ARG, "null manager");
    if (!m->committed) return pa::report(PA_ERR_INVALID_ARG, "commit the scheduled step first");
    auto it = m->reqs.find(parent);
    if (it == m->reqs.end() || !it->second->running)
        return pa::report(PA_ERR_INVALID_ARG, "request %lld is not running", (long long)parent);
    if (m->reqs.count(child)) return pa::report(PA_ERR_INVALID_ARG, "request %lld exists", (long long)child);
    if ((int32_t)m->running.size() >= m->max_num_seqs)
        return pa::report(PA_ERR_INVALID_ARG, "already %d running requests", m->max_num_seqs);
    const Request* p = it->second.get();
    auto r = std::make_unique<Request>(*p);
    r->id = child;
    for (int32_t b : r->blocks) ++m->blocks[b].ref;     // every block shared until one side writes
    m->running.push_back(r.get());
    m->reqs.emplace(child, std::move(r));
    return pa::report_ok();
}

pa_status pa_kvm_finish(pa_kvm* m, int64_t id) {
    if (!m) return pa::report(PA_ERR_INVALID_ARG, "null manager");
    auto it = m->reqs.find(id);
    if (it == m->reqs.end()) return pa::report(PA_ERR_INVALID_ARG, "no request %lld", (long long)id);
    if (!m->committed) return pa::report(PA_ERR_INVALID_ARG, "commit the scheduled step first");
    Request* r = it->second.get();
    m->free_blocks(r);
    m->running.erase(std::remove(m->running.begin(), m->running.end(), r), m->running.end());
    m->waiting.erase(std::remove(m->waiting.begin(), m->waiting.end(), r), m->waiting.end());
    m->reqs.erase(it);
    return pa::report_ok();
}

pa_status pa_kvm_schedule(pa_kvm* m, pa_kvm_step* out) {
    if (!m || !out) return pa::report(PA_ERR_INVALID_ARG, "null pointer");
    if (!m->committed) return pa::report(PA_ERR_INVALID_ARG, "commit the scheduled step first");
    m->sched.clear();
    m->out_preempted.clear();
    m->end_step();                                       // an empty previous step's marks
    m->out_copies.clear();
    int32_t budget = m->max_batched_tokens;

    // running requests first, in arrival order
    for (size_t i = 0; i < m->running.size() && budget > 0;) {
        Request* r = m->running[i];
        int32_t count = std::min<int32_t>((int32_t)r->tokens.size() - r->num_computed, budget);
        count = std::min(count, m->max_model_len - r->num_computed);
        if (count <= 0) {
            ++i;
            continue;
        }
        bool self_preempted = false;
        while (!m->reserve(r, r->num_computed, count, m->out_copies)) {
            // the newest running request: never one already scheduled this
            // step, since those come before r in the list
            Request* victim = m->running.back();
            m->running.pop_back();
            m->preempt(victim);
            if (victim == r) {
                self_preempted = true;
                break;
            }
        }
        if (self_preempted) break;
        m->sched.push_back({r, r->num_computed, count});
        budget -= count;
        ++i;
    }

    // then waiting requests, first come first served, unless this step preempted
    while (m->out_preempted.empty() && !m->waiting.empty() && budget > 0 &&
           (int32_t)m->running.size() < m->max_num_seqs) {
        Request* r = m->waiting.front();
        if (r->num_computed == 0 && r->blocks.empty()) m->acquire_prefix(r);
        int32_t count = std::min<int32_t>((int32_t)r->tokens.size() - r->num_computed, budget);
        count = std::min(count, m->max_model_len - r->num_computed);
        if (count <= 0 || !m->reserve(r, r->num_computed, count, m->out_copies)) {
            m->free_blocks(r);                             // give the prefix hits back
            r->num_computed = 0;
            break;
        }
        m->waiting.pop_front();
        r->running = true;
        m->running.push_back(r);
        m->sched.push_back({r, r->num_computed, count});
        budget -= count;
    }

    // the step's arrays
    // rows as long as the longest block list of the step (a valid row stride
    // for the kernels: every request's blocks cover its seq_len)
    const int32_t n = (int32_t)m->sched.size();
    int32_t W = 1;
    for (const Scheduled& sc : m->sched) W = std::max(W, (int32_t)sc.req->blocks.size());
    m->out_ids.assign(n, 0);
    m->out_qlen.assign(n, 0);
    m->out_cu.assign(n + 1, 0);
    m->out_seqlen.assign(n, 0);
    m->out_table.resize((size_t)n * W);
    m->out_tokens.clear();
    m->out_pos.clear();
    m->out_slots.clear();
    for (int32_t i = 0; i < n; ++i) {
        const Scheduled& s = m->sched[i];
        m->out_ids[i] = s.req->id;
        m->out_qlen[i] = s.count;
        m->out_cu[i + 1] = m->out_cu[i] + s.count;
        m->out_seqlen[i] = s.start + s.count;
        auto row = m->out_table.begin() + (size_t)i * W;
        std::fill(std::copy(s.req->blocks.begin(), s.req->blocks.end(), row), row + W, -1);
        for (int32_t p = s.start; p < s.start + s.count; ++p) {
            m->out_tokens.push_back(s.req->tokens[p]);
            m->out_pos.push_back(p);
            m->out_slots.push_back((int64_t)s.req->blocks[p / kBlockSize] * kBlockSize + p % kBlockSize);
        }
    }
    out->num_seqs = n;
    out->num_tokens = m->out_cu[n];
    out->max_blocks_per_req = W;
    out->request_ids = m->out_ids.data();
    out->query_lens = m->out_qlen.data();
    out->cu_query_lens = m->out_cu.data();
    out->seq_lens = m->out_seqlen.data();
    out->block_table = m->out_table.data();
    out->token_ids = m->out_tokens.data();
    out->positions = m->out_pos.data();
    out->slot_mapping = m->out_slots.data();
    out->copy_pairs = m->out_copies.data();
    out->num_copies = (int32_t)(m->out_copies.size() / 2);
    out->preempted = m->out_preempted.data();
    out->num_preempted = (int32_t)m->out_preempted.size();
    m->committed = n == 0;
    return pa::report_ok();
}

pa_status pa_kvm_commit(pa_kvm* m, const int32_t* next_tokens, int32_t n) {
    if (!m) return pa::report(PA_ERR_INVALID_ARG, "null manager");
    if (m->committed) {                                  // nothing scheduled: only an empty commit
        if (n == 0) return pa::report_ok();
        return pa::report(PA_ERR_INVALID_ARG, "no scheduled step to commit");
    }
    if (n != (int32_t)m->sched.size() || (n > 0 && !next_tokens))
        return pa::report(PA_ERR_INVALID_ARG, "%d next tokens for %zu scheduled requests", n, m->sched.size());
    for (int32_t i = 0; i < n; ++i) {
        Request* r = m->sched[i].req;
        r->num_computed = m->sched[i].start + m->sched[i].count;
        m->register_full(r);
        if (r->num_computed == (int32_t)r->tokens.size() && next_tokens[i] >= 0 &&
            (int32_t)r->tokens.size() < m->max_model_len)
            r->tokens.push_back(next_tokens[i]);
    }
    m->sched.clear();
    m->end_step();
    m->committed = true;
    return pa::report_ok();
}

int32_t pa_kvm_num_free_blocks(const pa_kvm* m) { return m ? m->num_free : -1; }

int32_t pa_kvm_num_cached_blocks(const pa_kvm* m) { return m ? (int32_t)m->cache.size() : -1; }

pa_status pa_kvm_request_info(const pa_kvm* m, int64_t id, int32_t* num_computed, int32_t* num_tokens,
                              int32_t* running, int32_t* blocks, int32_t blocks_cap, int32_t* num_blocks) {
    if (!m) return pa::report(PA_ERR_INVALID_ARG, "null manager");
    auto it = m->reqs.find(id);
    if (it == m->reqs.end()) return pa::report(PA_ERR_INVALID_ARG, "no request %lld", (long long)id);
    const Request* r = it->second.get();
    if (num_computed) *num_computed = r->num_computed;
    if (num_tokens) *num_tokens = (int32_t)r->tokens.size();
    if (running) *running = r->running ? 1 : 0;
    if (num_blocks) *num_blocks = (int32_t)r->blocks.size();
    if (blocks)
        for (int32_t i = 0; i < std::min<int32_t>(blocks_cap, (int32_t)r->blocks.size()); ++i) blocks[i] = r->blocks[i];
    return pa::report_ok();
}

int32_t pa_kvm_block_ref(const pa_kvm* m, int32_t block) {
    if (!m || block < 0 || block >= m->num_blocks) return -1;
    return m->blocks[block].ref;
}

}  // extern "C"
