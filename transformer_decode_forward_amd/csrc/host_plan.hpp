// Host-side bookkeeping of a decode call: batch intake and defaults, ubatch
// split and KV-cell placement.  Pure C++ (no HIP) so that it is the same code
// whether or not a device is present.
//
// Intake follows llama.cpp walkthrough "Step 10: forming the batch for one
// call": token ids in [0, n_vocab); absent sequence ids mean sequence 0;
// absent positions continue each sequence at seq_pos_max(s)+1 in batch
// order; absent output flags select the last token (or all with
// output_all).  ubatches are consecutive chunks of at most n_ubatch tokens
// ("Steps 11-12").  Cells: Ollama engine page "KV Cache: memory for causal
// attention" -- find contiguous slots, record position and sequences per
// cell.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "tdf.h"

namespace tdf {

constexpr int kMaxSeq = 64;

// One validated batch with every field filled in.
struct Intake {
  int n_tokens = 0;
  std::vector<int32_t> token, pos, seq0;     // seq0 = first sequence id of the token
  std::vector<uint64_t> seq_mask;            // every sequence of the token
  std::vector<int8_t> output;                // 1 = logits wanted
};

// KV-cell state: per-cell position and sequence mask, per-sequence list of
// cells in position order (append-only until clear).
class KvBook {
 public:
  void init(int n_ctx, int n_seq_max);
  void clear();

  int n_ctx() const { return n_ctx_; }
  int n_seq_max() const { return n_seq_max_; }
  int n_free() const { return n_ctx_ - n_used_; }
  int32_t seq_pos_max(int s) const { return seq_max_[s]; }
  int32_t cell_pos(int c) const { return cell_pos_[c]; }
  uint64_t cell_seq(int c) const { return cell_seq_[c]; }
  const std::vector<int32_t>& seq_cells(int s) const { return seq_cells_[s]; }

  // First run of n consecutive free cells scanning from cell 0; if there is
  // none, the n lowest-index free cells.  False if fewer than n are free.
  bool find_slots(int n, std::vector<int32_t>& out) const;

  // Remove sequence s from its cells with position in [p0, p1) (p1 < 0: no
  // upper end); cells left with no sequence become free.  The list of s is
  // compacted in order.  Arguments are checked by the caller.
  void seq_rm(int s, int32_t p0, int32_t p1);

  // Cells of sequence s with position in [p0, p1) (p1 < 0: no upper end)
  // that a shift by delta would move, in list order; false (and nothing
  // returned) if the shift is not allowed: a cell also holds another
  // sequence, a position would become negative, or s's positions would lose
  // their list order.
  bool shift_cells(int s, int32_t p0, int32_t p1, int32_t delta, std::vector<int32_t>& cells) const;
  // Apply a shift that shift_cells allowed.
  void seq_shift(int s, int32_t delta, const std::vector<int32_t>& cells);

  // Index in sequence s's list of its first cell with position >= pos_lo,
  // searching the first n entries (the list is position-ordered).
  int32_t first_at_or_after(int s, int32_t n, int32_t pos_lo) const;

  // Mark `cell` as holding (pos, seq_mask) and append it to each of its
  // sequences' lists; returns the cell's index in the list of sequence s0.
  int32_t place(int32_t cell, int32_t pos, uint64_t seq_mask, int s0,
                std::vector<int64_t>* list_writes);

 private:
  int n_ctx_ = 0, n_seq_max_ = 0, n_used_ = 0;
  std::vector<int32_t> cell_pos_;
  std::vector<uint64_t> cell_seq_;
  std::vector<int32_t> seq_max_;
  std::vector<std::vector<int32_t>> seq_cells_;
  int32_t first_free_hint_ = 0;
};

// Validate `b` and fill defaults.  Returns TDF_OK or TDF_E_INVALID (with a
// message in err); never changes `book`.
int intake_batch(const KvBook& book, const tdf_batch* b, int n_vocab, int n_batch,
                 bool output_all, Intake& out, std::string& err);

}  // namespace tdf
