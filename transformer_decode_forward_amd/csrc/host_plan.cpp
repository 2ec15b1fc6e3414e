// Batch intake and KV-cell bookkeeping (see host_plan.hpp for the sources).
#include "host_plan.hpp"

#include <algorithm>
#include <cstdio>

namespace tdf {

void KvBook::init(int n_ctx, int n_seq_max) {
  n_ctx_ = n_ctx;
  n_seq_max_ = n_seq_max;
  cell_pos_.assign(n_ctx, -1);
  cell_seq_.assign(n_ctx, 0);
  seq_max_.assign(n_seq_max, -1);
  seq_cells_.assign(n_seq_max, {});
  n_used_ = 0;
  first_free_hint_ = 0;
}

void KvBook::clear() { init(n_ctx_, n_seq_max_); }

bool KvBook::find_slots(int n, std::vector<int32_t>& out) const {
  out.clear();
  if (n <= 0 || n > n_free()) return false;
  // first run of n consecutive free cells; cells below the hint are all used
  int run_start = -1, run_len = 0;
  for (int c = first_free_hint_; c < n_ctx_; ++c) {
    if (cell_pos_[c] < 0) {
      if (run_len == 0) run_start = c;
      if (++run_len == n) {
        for (int i = 0; i < n; ++i) out.push_back(run_start + i);
        return true;
      }
    } else {
      run_len = 0;
    }
  }
  // no run long enough: the n lowest-index free cells
  for (int c = first_free_hint_; c < n_ctx_ && (int)out.size() < n; ++c)
    if (cell_pos_[c] < 0) out.push_back(c);
  return (int)out.size() == n;
}

int32_t KvBook::place(int32_t cell, int32_t pos, uint64_t seq_mask, int s0,
                      std::vector<int64_t>* list_writes) {
  cell_pos_[cell] = pos;
  cell_seq_[cell] = seq_mask;
  ++n_used_;
  while (first_free_hint_ < n_ctx_ && cell_pos_[first_free_hint_] >= 0) ++first_free_hint_;
  int32_t idx0 = -1;
  for (int s = 0; s < n_seq_max_; ++s) {
    if (!((seq_mask >> s) & 1)) continue;
    auto& lst = seq_cells_[s];
    int32_t idx = (int32_t)lst.size();
    lst.push_back(cell);
    seq_max_[s] = std::max(seq_max_[s], pos);
    if (list_writes) {
      list_writes->push_back((int64_t)s * n_ctx_ + idx);
      list_writes->push_back(cell);
    }
    if (s == s0) idx0 = idx;
  }
  return idx0;
}

int intake_batch(const KvBook& book, const tdf_batch* b, int n_vocab, int n_batch,
                 bool output_all, Intake& out, std::string& err) {
  char msg[160];
  if (!b) { err = "batch is NULL"; return TDF_E_INVALID; }
  const int n = b->n_tokens;
  if (n <= 0) { err = "n_tokens must be > 0"; return TDF_E_INVALID; }
  if (n > n_batch) {
    snprintf(msg, sizeof msg, "n_tokens %d exceeds n_batch %d", n, n_batch);
    err = msg;
    return TDF_E_INVALID;
  }
  if (!b->token) { err = "token array is NULL"; return TDF_E_INVALID; }
  out = Intake();
  out.n_tokens = n;
  out.token.assign(b->token, b->token + n);
  for (int i = 0; i < n; ++i) {
    if (out.token[i] < 0 || out.token[i] >= n_vocab) {
      snprintf(msg, sizeof msg, "invalid token[%d] = %d", i, out.token[i]);
      err = msg;
      return TDF_E_INVALID;
    }
  }
  const int n_seq_max = book.n_seq_max();
  out.seq0.resize(n);
  out.seq_mask.resize(n);
  if ((b->seq_id == nullptr) != (b->n_seq_id == nullptr)) {
    err = "seq_id and n_seq_id must both be given or both be NULL";
    return TDF_E_INVALID;
  }
  for (int i = 0; i < n; ++i) {
    if (!b->seq_id) {
      out.seq0[i] = 0;
      out.seq_mask[i] = 1;
      continue;
    }
    int k = b->n_seq_id[i];
    if (k < 1 || k > n_seq_max || !b->seq_id[i]) {
      snprintf(msg, sizeof msg, "invalid n_seq_id[%d] = %d", i, k);
      err = msg;
      return TDF_E_INVALID;
    }
    uint64_t m = 0;
    for (int j = 0; j < k; ++j) {
      int s = b->seq_id[i][j];
      if (s < 0 || s >= n_seq_max || ((m >> s) & 1)) {
        snprintf(msg, sizeof msg, "invalid seq_id[%d][%d] = %d", i, j, s);
        err = msg;
        return TDF_E_INVALID;
      }
      m |= 1ull << s;
    }
    out.seq0[i] = b->seq_id[i][0];
    out.seq_mask[i] = m;
  }
  // positions: running last position per sequence, cache first then batch
  int32_t last[kMaxSeq];
  for (int s = 0; s < n_seq_max; ++s) last[s] = book.seq_pos_max(s);
  out.pos.resize(n);
  for (int i = 0; i < n; ++i) {
    int32_t p = b->pos ? b->pos[i] : last[out.seq0[i]] + 1;
    if (p < 0) {
      snprintf(msg, sizeof msg, "invalid pos[%d] = %d", i, p);
      err = msg;
      return TDF_E_INVALID;
    }
    for (int s = 0; s < n_seq_max; ++s) {
      if (((out.seq_mask[i] >> s) & 1) && p <= last[s]) {
        snprintf(msg, sizeof msg, "pos[%d] = %d does not follow position %d of sequence %d", i, p,
                 last[s], s);
        err = msg;
        return TDF_E_INVALID;
      }
    }
    for (int s = 0; s < n_seq_max; ++s)
      if ((out.seq_mask[i] >> s) & 1) last[s] = p;
    out.pos[i] = p;
  }
  out.output.assign(n, 0);
  if (b->logits) {
    for (int i = 0; i < n; ++i) out.output[i] = b->logits[i] != 0;
  } else if (output_all) {
    std::fill(out.output.begin(), out.output.end(), 1);
  } else {
    out.output[n - 1] = 1;
  }
  return TDF_OK;
}

int32_t KvBook::first_at_or_after(int s, int32_t n, int32_t pos_lo) const {
  const std::vector<int32_t>& L = seq_cells_[s];
  int32_t lo = 0, hi = std::min<int32_t>(n, (int32_t)L.size());
  while (lo < hi) {
    const int32_t mid = (lo + hi) / 2;
    if (cell_pos_[L[mid]] < pos_lo) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

void KvBook::seq_rm(int s, int32_t p0, int32_t p1) {
  auto& lst = seq_cells_[s];
  std::vector<int32_t> keep;
  keep.reserve(lst.size());
  const uint64_t bit = 1ull << s;
  for (int32_t c : lst) {
    const int32_t p = cell_pos_[c];
    if (p >= p0 && (p1 < 0 || p < p1)) {
      cell_seq_[c] &= ~bit;
      if (cell_seq_[c] == 0) {
        cell_pos_[c] = -1;
        --n_used_;
        first_free_hint_ = std::min(first_free_hint_, c);
      }
    } else {
      keep.push_back(c);
    }
  }
  lst.swap(keep);
  seq_max_[s] = lst.empty() ? -1 : cell_pos_[lst.back()];
}

bool KvBook::shift_cells(int s, int32_t p0, int32_t p1, int32_t delta, std::vector<int32_t>& cells) const {
  cells.clear();
  const auto& lst = seq_cells_[s];
  const uint64_t bit = 1ull << s;
  int64_t prev = -1;  // new position of the previous list entry
  for (int32_t c : lst) {
    const int32_t p = cell_pos_[c];
    const bool hit = p >= p0 && (p1 < 0 || p < p1);
    const int64_t np = (int64_t)p + (hit ? delta : 0);
    if (hit) {
      if (cell_seq_[c] != bit) { cells.clear(); return false; }
      cells.push_back(c);
    }
    if (np < 0 || np <= prev || np > INT32_MAX) { cells.clear(); return false; }
    prev = np;
  }
  return true;
}

void KvBook::seq_shift(int s, int32_t delta, const std::vector<int32_t>& cells) {
  for (int32_t c : cells) cell_pos_[c] += delta;
  const auto& lst = seq_cells_[s];
  seq_max_[s] = lst.empty() ? -1 : cell_pos_[lst.back()];
}

}  // namespace tdf
