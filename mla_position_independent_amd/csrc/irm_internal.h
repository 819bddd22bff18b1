// Internal layout shared by the host table builder and the HIP kernels.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "irm.h"

namespace irm {

// One entry of the device chunk table (32 bytes).
struct DevEntry {
  uint32_t pool_row;  // first pool row of the entry
  uint32_t len;       // rows
  int32_t p_src;
  int32_t p_tgt;      // position of row 0 within its sequence
  uint32_t flags;
  uint32_t seq;       // owning sequence
  uint32_t out_row;   // assembled row of row 0: seq_base[seq] + p_tgt
  int32_t delta;      // p_tgt - p_src, forced to 0 for fresh entries
};
static_assert(sizeof(DevEntry) == 32, "device entry is 32 bytes");

// Rows per block of the block map: block_map[b] is the entry that holds
// assembled row b * kBlockRows.  A row's entry is found by walking forward
// from its block's entry.
constexpr uint32_t kBlockRows = 32;
constexpr uint32_t kPairs = IRM_D_ROPE / 2;  // 32 rotation pairs
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Device image: [entries | seq_first | seq_base | block_map | trig | rowmap].
// The host copies everything before trig; trig (float2 cos/sin per entry and
// pair) and the row map (16-byte {pool row, delta, entry, 0} record per
// assembled row, plus 64 records of padding) are computed on the GPU.
struct ImageLayout {
  size_t off_entries = 0, off_seq_first = 0, off_seq_base = 0, off_block_map = 0;
  size_t off_trig = 0, off_rowmap = 0, bytes = 0;
};

}  // namespace irm

struct irm_table {
  uint32_t n_seq = 0, n_chunks = 0;
  uint64_t total_rows = 0;
  uint32_t max_seq_len = 0;
  uint32_t min_seq_len = 0;
  uint64_t pool_rows = 0;       // pool size the table was validated against
  uint32_t n_blocks = 0;
  std::vector<irm::DevEntry> entries;
  std::vector<uint32_t> seq_first, seq_base, block_map;
  irm::ImageLayout layout;
  std::vector<unsigned char> image;  // host image of everything before trig
  void* dev = nullptr;               // device image after upload
  double inv_freq[32] = {};          // RoPE frequencies of the last upload / set_rope
};

namespace irm {
void set_error(const std::string& msg);
irm_status fail(irm_status st, const std::string& msg);
}  // namespace irm
