// Host-side block pool bookkeeping (spindle, "Paging"): a pool of fixed-size
// blocks, a per-sequence block table, reference counts and copy-on-write
// forking.  Pure host code; no GPU call.  Semantics are documented in
// include/pkv_block_manager.h.

#include <algorithm>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv_block_manager.h"

struct pkv_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 16;
  std::deque<int32_t> free_list;
  std::vector<int32_t> refcount;
  std::unordered_map<int32_t, std::vector<int32_t>> tables;
  int32_t next_seq = 0;

  int32_t take() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    refcount[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--refcount[b] == 0) free_list.push_back(b);
  }
};

namespace {

std::vector<int32_t>* find_table(pkv_bm* bm, int32_t seq) {
  auto it = bm->tables.find(seq);
  return it == bm->tables.end() ? nullptr : &it->second;
}

const std::vector<int32_t>* find_table(const pkv_bm* bm, int32_t seq) {
  auto it = bm->tables.find(seq);
  return it == bm->tables.end() ? nullptr : &it->second;
}

}  // namespace

extern "C" int pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                             pkv_bm** out) {
  if (!out) return PKV_ERR_NULL;
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0) return PKV_ERR_SHAPE;
  pkv_bm* bm = new (std::nothrow) pkv_bm();
  if (!bm) return PKV_ERR_DEVICE;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->refcount.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return PKV_ERR_ARG;
      }
      seen[b] = 1;
      bm->free_list.push_back(b);
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) bm->free_list.push_back(i);
  }
  *out = bm;
  return PKV_OK;
}

extern "C" void pkv_bm_destroy(pkv_bm* bm) { delete bm; }

extern "C" int pkv_bm_add_sequence(pkv_bm* bm, int32_t* seq_out) {
  if (!bm || !seq_out) return PKV_ERR_NULL;
  const int32_t id = bm->next_seq++;
  bm->tables.emplace(id, std::vector<int32_t>());
  *seq_out = id;
  return PKV_OK;
}

extern "C" int pkv_bm_prepare_write(pkv_bm* bm, int32_t seq, int32_t start, int32_t n,
                                    int32_t* copy_src, int32_t* copy_dst, int32_t copy_cap,
                                    int32_t* n_copies) {
  if (!bm || !n_copies) return PKV_ERR_NULL;
  *n_copies = 0;
  std::vector<int32_t>* table = find_table(bm, seq);
  if (!table || start < 0 || n < 0) return PKV_ERR_ARG;
  if (n == 0) return PKV_OK;
  const int64_t first = start / bm->block_size;
  const int64_t last = (static_cast<int64_t>(start) + n - 1) / bm->block_size;
  if (first > static_cast<int64_t>(table->size())) return PKV_ERR_ARG;  // would leave a hole
  // All or nothing: count fresh blocks and copies first.
  int64_t need = 0, copies = 0;
  for (int64_t j = first; j <= last; ++j) {
    if (j >= static_cast<int64_t>(table->size())) {
      ++need;
    } else if (bm->refcount[(*table)[j]] > 1) {
      ++need;
      ++copies;
    }
  }
  if (need > static_cast<int64_t>(bm->free_list.size())) return PKV_ERR_OUT_OF_BLOCKS;
  if (copies > 0 && (!copy_src || !copy_dst)) return PKV_ERR_NULL;
  if (copies > copy_cap) return PKV_ERR_ARG;
  int32_t k = 0;
  for (int64_t j = first; j <= last; ++j) {
    if (j >= static_cast<int64_t>(table->size())) {
      table->push_back(bm->take());
    } else if (bm->refcount[(*table)[j]] > 1) {
      const int32_t old = (*table)[j];
      const int32_t fresh = bm->take();
      copy_src[k] = old;
      copy_dst[k] = fresh;
      ++k;
      bm->drop(old);
      (*table)[j] = fresh;
    }
  }
  *n_copies = k;
  return PKV_OK;
}

extern "C" int pkv_bm_prepare_step(pkv_bm* bm, const int32_t* seqs, const int32_t* starts,
                                   const int32_t* counts, int32_t nseq, int32_t* tables,
                                   int32_t width, int32_t pad_id, int32_t* copy_src,
                                   int32_t* copy_dst, int32_t copy_cap, int32_t* n_copies,
                                   int32_t* n_done) {
  if (!bm || !seqs || !starts || !counts || !n_copies || !n_done) return PKV_ERR_NULL;
  if (nseq < 0 || copy_cap < 0) return PKV_ERR_ARG;
  *n_copies = 0;
  *n_done = 0;
  for (int32_t r = 0; r < nseq; ++r) {
    int32_t k = 0;
    const int st = pkv_bm_prepare_write(bm, seqs[r], starts[r], counts[r],
                                        copy_src ? copy_src + *n_copies : nullptr,
                                        copy_dst ? copy_dst + *n_copies : nullptr,
                                        copy_cap - *n_copies, &k);
    if (st != PKV_OK) return st;
    *n_copies += k;
    *n_done = r + 1;
  }
  return tables ? pkv_bm_fill_tables(bm, seqs, nseq, tables, width, pad_id) : PKV_OK;
}

extern "C" int pkv_bm_fork(pkv_bm* bm, int32_t parent, int32_t* child_out) {
  if (!bm || !child_out) return PKV_ERR_NULL;
  const std::vector<int32_t>* ptable = find_table(bm, parent);
  if (!ptable) return PKV_ERR_ARG;
  std::vector<int32_t> copy = *ptable;
  for (int32_t b : copy) ++bm->refcount[b];
  const int32_t id = bm->next_seq++;
  bm->tables.emplace(id, std::move(copy));
  *child_out = id;
  return PKV_OK;
}

extern "C" int pkv_bm_free_sequence(pkv_bm* bm, int32_t seq) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->tables.find(seq);
  if (it == bm->tables.end()) return PKV_ERR_ARG;
  for (int32_t b : it->second) bm->drop(b);
  bm->tables.erase(it);
  return PKV_OK;
}

extern "C" int pkv_bm_num_blocks_of(const pkv_bm* bm, int32_t seq, int32_t* n) {
  if (!bm || !n) return PKV_ERR_NULL;
  const std::vector<int32_t>* t = find_table(bm, seq);
  if (!t) return PKV_ERR_ARG;
  *n = static_cast<int32_t>(t->size());
  return PKV_OK;
}

extern "C" int pkv_bm_fill_tables(const pkv_bm* bm, const int32_t* seqs, int32_t nseq,
                                  int32_t* tables, int32_t width, int32_t pad_id) {
  if (!bm || (nseq > 0 && (!seqs || !tables))) return PKV_ERR_NULL;
  if (nseq < 0 || width < 0) return PKV_ERR_SHAPE;
  for (int32_t r = 0; r < nseq; ++r) {
    const std::vector<int32_t>* t = find_table(bm, seqs[r]);
    if (!t) return PKV_ERR_ARG;
    if (static_cast<int64_t>(t->size()) > width) return PKV_ERR_SHAPE;
  }
  for (int32_t r = 0; r < nseq; ++r) {
    const std::vector<int32_t>& t = *find_table(bm, seqs[r]);
    int32_t* row = tables + static_cast<int64_t>(r) * width;
    std::copy(t.begin(), t.end(), row);
    std::fill(row + t.size(), row + width, pad_id);
  }
  return PKV_OK;
}

extern "C" int pkv_bm_refcount(const pkv_bm* bm, int32_t block, int32_t* count) {
  if (!bm || !count) return PKV_ERR_NULL;
  if (block < 0 || block >= bm->num_blocks) return PKV_ERR_ARG;
  *count = bm->refcount[block];
  return PKV_OK;
}

extern "C" int pkv_bm_num_free(const pkv_bm* bm, int32_t* n) {
  if (!bm || !n) return PKV_ERR_NULL;
  *n = static_cast<int32_t>(bm->free_list.size());
  return PKV_OK;
}

extern "C" int pkv_bm_free_list(const pkv_bm* bm, int32_t* ids, int32_t cap, int32_t* n) {
  if (!bm || !n) return PKV_ERR_NULL;
  *n = static_cast<int32_t>(bm->free_list.size());
  if (cap < *n) return *n == 0 ? PKV_OK : (ids ? PKV_ERR_ARG : PKV_ERR_NULL);
  if (*n > 0 && !ids) return PKV_ERR_NULL;
  std::copy(bm->free_list.begin(), bm->free_list.end(), ids);
  return PKV_OK;
}
