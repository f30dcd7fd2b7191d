// Host-side manager of a KV page pool reserved once.
//
// The pool of num_blocks pages is sized once, when serving starts, and serves
// every request; its page count is what admission is checked against, so a
// burst of requests changes the queue, not the memory footprint (vllm-metal
// v0.4.0 release post, "Set a predictable memory budget").  Sequences that
// share a prefix hold the same physical pages (a reference count per page);
// a sequence about to write into a page it shares first gets a private copy
// of that page (copy-on-write), so shared pages are only ever read ("Prefix
// caching on hybrid models": rows are written in place into the pool, never
// by copying the pool).
//
// The manager only does the bookkeeping on the host: it hands out slots for
// the step's new rows (the slot_mapping of pkv_append), block-table rows and
// lengths (for pkv_attention), and the list of page copies a copy-on-write
// needs, which the caller performs on the device with pkv_copy_blocks before
// the step's append.  It is not thread-safe: one host thread drives a pool.
#pragma once

#include <cstdint>
#include <vector>

namespace pkv {

class PagePool {
public:
    // Result codes of the operations below (mapped onto PKV_* by the C ABI).
    enum Status { kOk = 0, kBadArg = 1, kNoMem = 2 };

    PagePool(int64_t num_blocks, int block_size, int max_seqs, int max_blocks_per_seq)
        : num_blocks_(num_blocks), bs_(block_size), max_seqs_(max_seqs),
          max_bps_(max_blocks_per_seq), ref_((size_t)num_blocks, 0), seqs_((size_t)max_seqs) {
        free_.reserve((size_t)num_blocks);
        // a stack: page 0 is handed out first
        for (int64_t b = num_blocks - 1; b >= 0; --b) free_.push_back((int32_t)b);
    }

    int64_t num_blocks() const { return num_blocks_; }
    int block_size() const { return bs_; }
    int max_seqs() const { return max_seqs_; }
    int max_blocks_per_seq() const { return max_bps_; }
    int64_t free_blocks() const { return (int64_t)free_.size(); }

    bool live(int seq) const { return valid(seq) && seqs_[(size_t)seq].live; }
    int64_t length(int seq) const { return live(seq) ? seqs_[(size_t)seq].len : -1; }
    int32_t refcount(int64_t block) const {
        return (block >= 0 && block < num_blocks_) ? ref_[(size_t)block] : -1;
    }
    const std::vector<int32_t>& pages(int seq) const { return seqs_[(size_t)seq].pages; }

    // Sets the order in which the free pages are handed out: order[0] first.
    // order must list every free page exactly once (a pool that has served
    // requests for a while hands out pages in no particular order; a caller
    // can reproduce that, or any placement, by a permutation of its own).
    Status set_free_order(const int32_t* order, int64_t n) {
        if (n != free_blocks() || (n > 0 && !order)) return kBadArg;
        std::vector<uint8_t> seen((size_t)num_blocks_, 0);
        for (int64_t i = 0; i < n; ++i) {
            const int32_t b = order[i];
            if (b < 0 || b >= num_blocks_ || ref_[(size_t)b] != 0 || seen[(size_t)b]) return kBadArg;
            seen[(size_t)b] = 1;
        }
        // free_ is a stack (back = next page handed out)
        for (int64_t i = 0; i < n; ++i) free_[(size_t)(n - 1 - i)] = order[i];
        return kOk;
    }

    // Pages a new sequence of num_tokens tokens needs now.
    int64_t pages_for(int64_t num_tokens) const { return (num_tokens + bs_ - 1) / bs_; }
    bool can_admit(int64_t num_tokens) const {
        return num_tokens >= 0 && pages_for(num_tokens) <= max_bps_ &&
               pages_for(num_tokens) <= free_blocks();
    }

    Status add_seq(int seq) {
        if (!valid(seq) || seqs_[(size_t)seq].live) return kBadArg;
        Seq& s = seqs_[(size_t)seq];
        s.live = true;
        s.len = 0;
        s.pages.clear();
        return kOk;
    }

    // child starts as the first `shared` tokens of parent, on parent's pages.
    Status fork(int parent, int child, int64_t shared) {
        if (!live(parent) || !valid(child) || seqs_[(size_t)child].live || parent == child)
            return kBadArg;
        const Seq& p = seqs_[(size_t)parent];
        if (shared < 0 || shared > p.len) return kBadArg;
        Seq& c = seqs_[(size_t)child];
        c.live = true;
        c.len = shared;
        c.pages.assign(p.pages.begin(), p.pages.begin() + pages_for(shared));
        for (int32_t b : c.pages) ++ref_[(size_t)b];
        return kOk;
    }

    // Slots for n new tokens of seq (slot = page * block_size + offset), in
    // token order.  If the sequence's last page is partly filled and shared,
    // it first moves to a private copy: (cow_src[i], cow_dst[i]) lists such
    // copies (at most one per call).  Nothing changes unless every page fits.
    Status append(int seq, int64_t n, int64_t* slots, int32_t* cow_src, int32_t* cow_dst,
                  int* num_cow) {
        if (num_cow) *num_cow = 0;
        if (!live(seq) || n < 0) return kBadArg;
        Seq& s = seqs_[(size_t)seq];
        const int64_t new_len = s.len + n;
        const int64_t need = pages_for(new_len);
        if (need > max_bps_) return kBadArg;
        const bool cow = n > 0 && s.len % bs_ != 0 && ref_[(size_t)s.pages.back()] > 1;
        const int64_t fresh = need - (int64_t)s.pages.size() + (cow ? 1 : 0);
        if (fresh > free_blocks()) return kNoMem;
        if (cow) {
            const int32_t src = s.pages.back();
            const int32_t dst = pop();
            --ref_[(size_t)src];
            s.pages.back() = dst;
            if (cow_src) cow_src[0] = src;
            if (cow_dst) cow_dst[0] = dst;
            if (num_cow) *num_cow = 1;
        }
        while ((int64_t)s.pages.size() < need) s.pages.push_back(pop());
        if (slots)
            for (int64_t i = 0; i < n; ++i) {
                const int64_t pos = s.len + i;
                slots[i] = (int64_t)s.pages[(size_t)(pos / bs_)] * bs_ + pos % bs_;
            }
        s.len = new_len;
        return kOk;
    }

    // Fresh pages append(seq, n) would take (with its copy-on-write page), or
    // -1 if the call is invalid.
    int64_t fresh_pages(int seq, int64_t n) const {
        if (!live(seq) || n < 0) return -1;
        const Seq& s = seqs_[(size_t)seq];
        const int64_t need = pages_for(s.len + n);
        if (need > max_bps_) return -1;
        const bool cow = n > 0 && s.len % bs_ != 0 && ref_[(size_t)s.pages.back()] > 1;
        return need - (int64_t)s.pages.size() + (cow ? 1 : 0);
    }

    // append() for several distinct sequences at once (one step of a serving
    // loop): slots are written back to back in the order given, copy-on-write
    // pairs to cow_src/cow_dst (room for n).  All-or-nothing: nothing changes
    // unless every sequence is valid and all the pages fit.
    Status append_batch(const int* seqs, const int64_t* counts, int n, int64_t* slots,
                        int32_t* cow_src, int32_t* cow_dst, int* num_cow) {
        if (num_cow) *num_cow = 0;
        int64_t total = 0;
        bool bad = false;
        for (int i = 0; i < n; ++i) {
            const int64_t f = fresh_pages(seqs[i], counts[i]);
            if (f < 0) {
                bad = true;  // invalid; marks are cleared below
                n = i;
                break;
            }
            Seq& s = seqs_[(size_t)seqs[i]];
            if (s.mark) bad = true;  // one entry per sequence
            s.mark = true;
            total += f;
        }
        for (int i = 0; i < n; ++i) seqs_[(size_t)seqs[i]].mark = false;
        if (bad) return kBadArg;
        if (total > free_blocks()) return kNoMem;
        int64_t at = 0;
        int nc = 0;
        for (int i = 0; i < n; ++i) {
            int c = 0;
            append(seqs[i], counts[i], slots ? slots + at : nullptr, cow_src ? cow_src + nc : nullptr,
                   cow_dst ? cow_dst + nc : nullptr, &c);
            at += counts[i];
            nc += c;
        }
        if (num_cow) *num_cow = nc;
        return kOk;
    }

    // Drops the tokens past new_len (rejected draft tokens of a verify
    // window); pages no longer needed are released.
    Status truncate(int seq, int64_t new_len) {
        if (!live(seq)) return kBadArg;
        Seq& s = seqs_[(size_t)seq];
        if (new_len < 0 || new_len > s.len) return kBadArg;
        const int64_t keep = pages_for(new_len);
        while ((int64_t)s.pages.size() > keep) {
            release(s.pages.back());
            s.pages.pop_back();
        }
        s.len = new_len;
        return kOk;
    }

    Status free_seq(int seq) {
        if (!live(seq)) return kBadArg;
        Seq& s = seqs_[(size_t)seq];
        for (int32_t b : s.pages) release(b);
        s.pages.clear();
        s.len = 0;
        s.live = false;
        return kOk;
    }

private:
    struct Seq {
        bool live = false;
        bool mark = false;  // append_batch: listed already
        int64_t len = 0;
        std::vector<int32_t> pages;
    };

    bool valid(int seq) const { return seq >= 0 && seq < max_seqs_; }
    int32_t pop() {
        const int32_t b = free_.back();
        free_.pop_back();
        ref_[(size_t)b] = 1;
        return b;
    }
    void release(int32_t b) {
        if (--ref_[(size_t)b] == 0) free_.push_back(b);
    }

    int64_t num_blocks_;
    int bs_;
    int max_seqs_;
    int max_bps_;
    std::vector<int32_t> ref_;   // sequences holding each page (0 = free)
    std::vector<int32_t> free_;  // free pages, used as a stack
    std::vector<Seq> seqs_;
};

}  // namespace pkv
