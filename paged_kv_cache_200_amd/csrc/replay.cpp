// Allocator replay (spindle, "Paging"): a request stream through a contiguous
// per-sequence allocator or through the block manager; see pkv_replay.h for the model.
// Host code only.

#include <algorithm>
#include <deque>
#include <map>
#include <vector>

#include "pkv_block_manager.h"
#include "pkv_replay.h"

namespace {

// First-fit allocator over one linear range of token slots: free runs keyed by their
// start, never adjacent (released runs merge with their neighbours).
class Arena {
 public:
  explicit Arena(int64_t total) { free_[0] = total; }

  bool alloc(int64_t size, int64_t* where) {
    for (auto it = free_.begin(); it != free_.end(); ++it) {
      if (it->second < size) continue;
      *where = it->first;
      const int64_t rest = it->second - size;
      const int64_t next = it->first + size;
      free_.erase(it);
      if (rest > 0) free_[next] = rest;
      return true;
    }
    return false;
  }

  void release(int64_t start, int64_t size) {
    auto it = free_.emplace(start, size).first;
    auto next = std::next(it);
    if (next != free_.end() && it->first + it->second == next->first) {
      it->second += next->second;
      free_.erase(next);
    }
    if (it != free_.begin()) {
      auto prev = std::prev(it);
      if (prev->first + prev->second == it->first) {
        prev->second += it->second;
        free_.erase(it);
      }
    }
  }

 private:
  std::map<int64_t, int64_t> free_;
};

struct Request {
  int64_t prompt = 0, gen = 0;
  int64_t length = 0;  // cached tokens while running
  int64_t start = 0;   // contiguous: reserved run
  int32_t seq = -1;    // paged: block-manager sequence
  bool admitted_now = false;
};

class Replay {
 public:
  Replay(int32_t policy, int64_t max_new, int64_t total, int32_t block_size,
         std::vector<Request> reqs)
      : policy_(policy), max_new_(max_new), block_(block_size), arena_(total),
        reqs_(std::move(reqs)) {}

  ~Replay() {
    if (bm_ != nullptr) pkv_bm_destroy(bm_);
  }

  int init(int64_t total) {
    if (policy_ == PKV_REPLAY_PAGED)
      return pkv_bm_create(static_cast<int32_t>(total / block_), block_, nullptr, &bm_);
    return PKV_OK;
  }

  // Runs the whole stream; step callback receives (slots, tokens, running) per step.
  template <typename F>
  int run(F&& on_step, pkv_replay_result* res) {
    std::deque<int> waiting;
    for (int r = 0; r < static_cast<int>(reqs_.size()); ++r) waiting.push_back(r);
    std::vector<int> running;  // admission order
    double util_sum = 0.0;
    res->peak_slots = 0;
    res->steps = 0;
    res->preemptions = 0;
    while (!waiting.empty() || !running.empty()) {
      ++res->steps;
      for (int r : running) reqs_[r].admitted_now = false;
      // Admission, FIFO, no overtaking.
      while (!waiting.empty()) {
        const int r = waiting.front();
        Request& q = reqs_[r];
        bool ok;
        int st = admit(q, &ok);
        if (st != PKV_OK) return st;
        if (!ok) break;
        waiting.pop_front();
        running.push_back(r);
        q.admitted_now = true;
        q.length = q.prompt + 1;
      }
      if (running.empty()) return PKV_ERR_SHAPE;  // cannot happen for fitting requests
      // One token for every request admitted earlier.
      for (size_t k = 0; k < running.size();) {
        Request& q = reqs_[running[k]];
        if (q.admitted_now) {
          ++k;
          continue;
        }
        if (policy_ == PKV_REPLAY_PAGED) {
          int32_t nb = 0;
          int st = pkv_bm_num_blocks_of(bm_, q.seq, &nb);
          if (st != PKV_OK) return st;
          if (q.length == static_cast<int64_t>(nb) * block_) {
            bool self = false;
            for (;;) {
              int32_t nfree = 0;
              st = pkv_bm_num_free(bm_, &nfree);
              if (st != PKV_OK) return st;
              if (nfree > 0) break;
              const int victim = running.back();
              running.pop_back();
              Request& v = reqs_[victim];
              st = pkv_bm_free_sequence(bm_, v.seq);
              if (st != PKV_OK) return st;
              v.seq = -1;
              v.length = 0;
              v.admitted_now = false;
              waiting.push_front(victim);
              ++res->preemptions;
              if (&v == &q) {
                self = true;
                break;
              }
            }
            if (self) continue;  // q was the last running request
            int32_t ncopy = 0;
            st = pkv_bm_prepare_write(bm_, q.seq, static_cast<int32_t>(q.length), 1, nullptr,
                                      nullptr, 0, &ncopy);
            if (st != PKV_OK) return st;
          }
        }
        ++q.length;
        ++k;
      }
      int64_t slots = 0, tokens = 0;
      for (int r : running) {
        const Request& q = reqs_[r];
        tokens += q.length;
        if (policy_ == PKV_REPLAY_CONTIGUOUS) {
          slots += q.prompt + max_new_;
        } else {
          int32_t nb = 0;
          const int st = pkv_bm_num_blocks_of(bm_, q.seq, &nb);
          if (st != PKV_OK) return st;
          slots += static_cast<int64_t>(nb) * block_;
        }
      }
      on_step(res->steps - 1, slots, tokens, static_cast<int32_t>(running.size()));
      res->peak_slots = std::max(res->peak_slots, slots);
      util_sum += slots > 0 ? static_cast<double>(tokens) / static_cast<double>(slots) : 0.0;
      // Requests that reached their length leave.
      std::vector<int> stay;
      stay.reserve(running.size());
      for (int r : running) {
        Request& q = reqs_[r];
        if (q.length != q.prompt + q.gen) {
          stay.push_back(r);
          continue;
        }
        if (policy_ == PKV_REPLAY_CONTIGUOUS) {
          arena_.release(q.start, q.prompt + max_new_);
        } else {
          const int st = pkv_bm_free_sequence(bm_, q.seq);
          if (st != PKV_OK) return st;
          q.seq = -1;
        }
      }
      running.swap(stay);
    }
    res->mean_utilisation = res->steps > 0 ? util_sum / res->steps : 0.0;
    return PKV_OK;
  }

 private:
  int admit(Request& q, bool* ok) {
    *ok = false;
    if (policy_ == PKV_REPLAY_CONTIGUOUS) {
      *ok = arena_.alloc(q.prompt + max_new_, &q.start);
      return PKV_OK;
    }
    int32_t nfree = 0;
    int st = pkv_bm_num_free(bm_, &nfree);
    if (st != PKV_OK) return st;
    const int64_t need = (q.prompt + 1 + block_ - 1) / block_;
    if (need > nfree) return PKV_OK;
    st = pkv_bm_add_sequence(bm_, &q.seq);
    if (st != PKV_OK) return st;
    int32_t ncopy = 0;
    st = pkv_bm_prepare_write(bm_, q.seq, 0, static_cast<int32_t>(q.prompt + 1), nullptr, nullptr,
                              0, &ncopy);
    if (st != PKV_OK) return st;
    *ok = true;
    return PKV_OK;
  }

  int32_t policy_;
  int64_t max_new_;
  int32_t block_;
  Arena arena_;
  pkv_bm* bm_ = nullptr;
  std::vector<Request> reqs_;
};

}  // namespace

extern "C" int pkv_replay_allocator(int32_t policy, int32_t num_requests,
                                    const int32_t* prompt_lens, const int32_t* gen_lens,
                                    int32_t max_new_tokens, int32_t total_slots,
                                    int32_t block_size, int64_t* slots_trace,
                                    int64_t* tokens_trace, int32_t* running_trace,
                                    int32_t trace_cap, pkv_replay_result* out) {
  if (out == nullptr) return PKV_ERR_NULL;
  if (policy != PKV_REPLAY_CONTIGUOUS && policy != PKV_REPLAY_PAGED) return PKV_ERR_ARG;
  if (num_requests < 0 || block_size <= 0 || total_slots <= 0 || max_new_tokens < 1 ||
      total_slots % block_size != 0 || trace_cap < 0)
    return PKV_ERR_SHAPE;
  if (num_requests > 0 && (prompt_lens == nullptr || gen_lens == nullptr)) return PKV_ERR_NULL;
  const bool traced = slots_trace != nullptr || tokens_trace != nullptr || running_trace != nullptr;
  if (traced && (slots_trace == nullptr || tokens_trace == nullptr || running_trace == nullptr))
    return PKV_ERR_NULL;
  std::vector<Request> reqs(static_cast<size_t>(num_requests));
  for (int32_t r = 0; r < num_requests; ++r) {
    Request& q = reqs[r];
    q.prompt = prompt_lens[r];
    q.gen = gen_lens[r];
    if (q.prompt < 0 || q.gen < 1 || q.gen > max_new_tokens) return PKV_ERR_SHAPE;
    // every request must fit an empty pool on its own
    if (policy == PKV_REPLAY_CONTIGUOUS && q.prompt + max_new_tokens > total_slots)
      return PKV_ERR_SHAPE;
    if (policy == PKV_REPLAY_PAGED &&
        (q.prompt + q.gen + block_size - 1) / block_size > total_slots / block_size)
      return PKV_ERR_SHAPE;
  }
  Replay rp(policy, max_new_tokens, total_slots, block_size, std::move(reqs));
  int st = rp.init(total_slots);
  if (st != PKV_OK) return st;
  return rp.run(
      [&](int32_t step, int64_t slots, int64_t tokens, int32_t running) {
        if (traced && step < trace_cap) {
          slots_trace[step] = slots;
          tokens_trace[step] = tokens;
          running_trace[step] = running;
        }
      },
      out);
}
