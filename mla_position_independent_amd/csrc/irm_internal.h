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

// The rotate-gather reads each pool row once per table however many entries
// place it: entries are grouped by their first pool row (a registry chunk
// reused by several requests), and a group is cut into records of at most
// kGroupRows rows and kGroupMembers members.  Every record lists its members
// (entry indices) and is worked on in items of kItemRows rows, each loaded
// once and written to every member.  Members may be shorter than the group (a truncated
// chunk): a member takes the rows below its own length.
struct GatherGroup {
  uint32_t pool_row;    // first pool row of the record
  uint32_t n_rows;      // rows of the record, at most kGroupRows
  uint32_t member_off;  // first member in the member list
  uint32_t n_members;
  uint32_t row_off;     // the record's first row within each member entry
  uint32_t item_off;    // first work item of the record
  uint32_t pad[2];
};
static_assert(sizeof(GatherGroup) == 32, "gather group record is 32 bytes");
constexpr uint32_t kGroupRows = 256;
constexpr uint32_t kGroupMembers = 8;
constexpr uint32_t kItemRows = 8;

// Rows per block of the block map: block_map[b] is the entry that holds
// assembled row b * kBlockRows.  A row's entry is found by walking forward
// from its block's entry.
constexpr uint32_t kBlockRows = 32;
constexpr uint32_t kPairs = IRM_D_ROPE / 2;  // 32 rotation pairs
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Device image: [entries | seq_first | seq_base | block_map | groups |
// members | trig | rowmap | items].  The host copies everything before trig;
// trig (float2 cos/sin per entry and pair), the row map (16-byte {pool row,
// delta, entry, 0} record per assembled row, plus 64 records of padding) and
// the gather items (16-byte {first pool row, rows | members << 4, first
// member, row offset} per item) are computed on the GPU.
struct ImageLayout {
  size_t off_entries = 0, off_seq_first = 0, off_seq_base = 0, off_block_map = 0;
  size_t off_groups = 0, off_members = 0;
  size_t off_trig = 0, off_rowmap = 0, off_items = 0, bytes = 0;
};

}  // namespace irm

struct irm_table {
  uint32_t n_seq = 0, n_chunks = 0;
  uint64_t total_rows = 0;
  uint32_t max_seq_len = 0;
  uint32_t min_seq_len = 0;
  uint64_t pool_rows = 0;       // pool size the table was validated against
  uint32_t n_blocks = 0;
  uint32_t n_groups = 0;        // gather group records
  uint64_t n_items = 0;         // gather work items
  uint64_t read_rows = 0;       // pool rows one rotate-gather reads (sum of record rows)
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
