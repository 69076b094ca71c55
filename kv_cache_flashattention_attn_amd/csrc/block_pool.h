// Host-side bookkeeping of a paged KV cache's physical blocks.
//
// The cache is cut into 16-token blocks; a per-sequence block table maps logical
// blocks to physical ones, and a finished sequence's blocks are reused at once
// ("KV Cache:推理慢的真正原因", 工程优化手段 / 1).  Blocks come from a free list
// and return to it when a sequence finishes ("KV缓存与Flash注意力", 练习, the hard
// exercise); a prompt's blocks can be shared by the completions that branch from
// it (the medium exercise there), with a holder count per block and copy on write
// of a shared, partly filled last block.
//
// Policy: the free list is a stack (block 0 on top initially; a freed block is
// pushed on top), so the most recently freed block is handed out first while it
// is still warm in the device's L2.  Every call validates its arguments fully
// before it changes anything: a failed call leaves the pool and the row as they
// were.
#pragma once

#include <cstdint>
#include <vector>

namespace attn {

constexpr int kPoolBlockTokens = 16;

inline int pool_blocks_for(int n_tokens) { return (n_tokens + kPoolBlockTokens - 1) / kPoolBlockTokens; }

struct BlockPool {
  std::vector<int32_t> free_stack;  // back() = top
  std::vector<int32_t> holders;

  explicit BlockPool(int n) : holders(n, 0) {
    free_stack.reserve(n);
    for (int b = n - 1; b >= 0; --b) free_stack.push_back(b);
  }

  int num_blocks() const { return static_cast<int>(holders.size()); }

  // true iff the row's first ceil(len/16) entries are held blocks
  bool row_ok(const int32_t* row, int len) const {
    const int nb = pool_blocks_for(len);
    for (int j = 0; j < nb; ++j) {
      const int32_t b = row[j];
      if (b < 0 || b >= num_blocks() || holders[b] == 0) return false;
    }
    return true;
  }

  int32_t take() {
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    holders[b] = 1;
    return b;
  }

  void drop(int32_t b) {
    if (--holders[b] == 0) free_stack.push_back(b);
  }
};

}  // namespace attn
