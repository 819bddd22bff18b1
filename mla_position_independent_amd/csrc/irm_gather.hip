// Table-derived device data and the standalone rotate-gather kernel.
//
// The rotate-gather assembles every sequence of a chunk table from the
// registry pool, applying k_r = R(p_tgt - p_src) k_r_base to hit rows and
// copying c_KV unchanged (Irminsul pages: gist.science summary, sections 2.1
// and 2.2; gentlecold.top article, sections 4, 5 and 15).

#include <hip/hip_runtime.h>

#include "irm_device.h"
#include "irm_launch.h"

namespace irm {
namespace {

using namespace irm::dev;

// ---------------------------------------------------------------------------
// trig prepass: cos/sin(delta_e * w_i) in double, stored as float2
// ---------------------------------------------------------------------------
__global__ void trig_kernel(const DevEntry* __restrict__ ents, uint32_t n_entries, InvFreq f,
                            float2* __restrict__ trig) {
  const uint32_t idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_entries * irm::kPairs) return;
  const uint32_t e = idx / irm::kPairs, i = idx % irm::kPairs;
  const double phi = (double)ents[e].delta * f.w[i];
  double s, c;
  sincos(phi, &s, &c);
  trig[idx] = make_float2((float)c, (float)s);
}

// ---------------------------------------------------------------------------
// gather index export
// ---------------------------------------------------------------------------
__global__ void gather_index_kernel(Image im, uint32_t total_rows, int64_t* __restrict__ pool_row,
                                    int32_t* __restrict__ delta) {
  const uint32_t g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= total_rows) return;
  const uint32_t e = find_entry(im, g);
  const DevEntry d = im.ents[e];
  if (pool_row) pool_row[g] = (int64_t)d.pool_row + (g - d.out_row);
  if (delta) delta[g] = d.delta;
}

// ---------------------------------------------------------------------------
// table prepare, three passes in one launch.  Row map: one 16-byte record
// per assembled row, {pool row, delta (0 if fresh), entry (kNoRot if delta
// is 0), 0}, followed by kTile records of {0, 0, kNoRot, 0} so that
// whole-tile reads never leave the array; the first map_blocks workgroups
// write it (one row per thread), the next trig_blocks the trig rows as
// trig_kernel does, the rest the rotate-gather's work items (one group
// record per thread, at most kGroupRows / kItemRows items each).  (Row map
// and trig in one launch: 11.8 us against 13.4 us for the 64 x 32768-token
// batch; four rows per thread with one entry lookup took 25 us.)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prepare_kernel(Image im, uint32_t total_rows, uint32_t map_blocks,
                                                      uint32_t trig_blocks, uint32_t n_groups, InvFreq f,
                                                      uint4* __restrict__ rowmap, float2* __restrict__ trig,
                                                      uint4* __restrict__ items) {
  if (blockIdx.x < map_blocks) {
    const uint32_t g = blockIdx.x * 256 + threadIdx.x;
    if (g >= total_rows + kTile) return;
    if (g >= total_rows) {
      rowmap[g] = make_uint4(0u, 0u, kNoRot, 0u);
      return;
    }
    const uint32_t e = find_entry(im, g);
    const DevEntry d = im.ents[e];
    rowmap[g] = make_uint4(d.pool_row + (g - d.out_row), (uint32_t)d.delta, d.delta != 0 ? e : kNoRot, 0u);
    return;
  }
  if (blockIdx.x < map_blocks + trig_blocks) {
    const uint32_t idx = (blockIdx.x - map_blocks) * 256 + threadIdx.x;
    if (idx >= im.n_entries * irm::kPairs) return;
    const uint32_t e = idx / irm::kPairs, i = idx % irm::kPairs;
    const double phi = (double)im.ents[e].delta * f.w[i];
    double sn, cn;
    sincos(phi, &sn, &cn);
    trig[idx] = make_float2((float)cn, (float)sn);
    return;
  }
  const uint32_t gi = (blockIdx.x - map_blocks - trig_blocks) * 256 + threadIdx.x;
  if (gi >= n_groups) return;
  const GatherGroup gr = im.groups[gi];
  for (uint32_t r = 0; r < gr.n_rows; r += kItemRows)
    items[gr.item_off + r / kItemRows] = make_uint4(gr.pool_row + r, min(kItemRows, gr.n_rows - r) | (gr.n_members << 4),
                                                    gr.member_off, gr.row_off + r);
}

// ---------------------------------------------------------------------------
// rotate-gather: one wave per work item of up to kItemRows rows of one
// group (entries that start at the same pool row, i.e. a registry chunk
// placed by several requests).  The wave loads the item's rows once and
// writes them to every member entry at that entry's assembled rows: slot i
// (i < 8) of lane l is c_KV unit l of row i (each load and store moves one
// whole 1 KB c_KV row), slot 8 is k_r unit l % 8 of row l / 8, turned by
// the member's own (cos, sin) row unless its delta is 0; a member shorter
// than the item takes the rows below its length.  Reading each distinct
// pool row once per table takes the chunk reuse across requests out of the
// HBM read stream: on the 64 x 32768-token batches the reads shrink to 62%
// (uniform chunk lengths) and 44% (CDC-like lengths) of one read per
// assembled row, while every assembled row is still written once; measured
// 0.737 and 0.673 ms per launch against 0.775 and 0.740 ms for a gather
// that reads every assembled row (one-wave workgroups of 4 units per lane
// over the row map).  Items run in the assembled order of their first
// member (the host orders the records so).  Loads go through the cache
// (non-temporal loads and four-row items measured within 1%), stores are
// non-temporal (every output line is written once).
// ---------------------------------------------------------------------------
constexpr int kGatherThreads = 64;
static_assert(kItemRows == 8 && kLatUnits == kGatherThreads, "one c_KV row per slot, eight k_r rows in one");

__global__ __launch_bounds__(kGatherThreads) void rotate_gather_kernel(Image im, const uint4* __restrict__ pool,
                                                                  uint4* __restrict__ out,
                                                                  float* __restrict__ kr_f32, uint32_t pool_last) {
  const uint4 it = im.items[blockIdx.x];
  const uint32_t rows = it.y & 15u, n_members = it.y >> 4, lane = threadIdx.x, kr_row = lane >> 3;
  const u32x4_t* P = reinterpret_cast<const u32x4_t*>(pool);
  u32x4_t* O = reinterpret_cast<u32x4_t*>(out);
  u32x4_t v[kItemRows + 1];
#pragma unroll
  for (uint32_t i = 0; i < kItemRows; ++i)
    if (i < rows) v[i] = P[(size_t)min(it.x + i, pool_last) * kUnitsPerRow + lane];
  if (kr_row < rows) v[kItemRows] = P[(size_t)min(it.x + kr_row, pool_last) * kUnitsPerRow + kLatUnits + (lane & 7)];
  for (uint32_t k = 0; k < n_members; ++k) {
    const uint32_t e = im.members[it.z + k];
    const DevEntry d = im.ents[e];
    if (d.len <= it.w) continue;
    const uint32_t mine = min(rows, d.len - it.w);
    const uint64_t dst0 = (uint64_t)d.out_row + it.w;  // assembled row of the item's row 0
#pragma unroll
    for (uint32_t i = 0; i < kItemRows; ++i)
      if (i < mine) __builtin_nontemporal_store(v[i], O + (dst0 + i) * kUnitsPerRow + lane);
    if (kr_row < mine) {
      const uint4 wu = __builtin_bit_cast(uint4, v[kItemRows]);
      float f[8];
      u32x4_t w = v[kItemRows];
      if (d.delta != 0) {
        rotate_unit_f32(wu, im.trig + (size_t)e * kPairs + (lane & 7) * 4, f);
        w = u32x4_t{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])};
      } else {
        f[0] = bf16_lo(wu.x); f[1] = bf16_hi(wu.x); f[2] = bf16_lo(wu.y); f[3] = bf16_hi(wu.y);
        f[4] = bf16_lo(wu.z); f[5] = bf16_hi(wu.z); f[6] = bf16_lo(wu.w); f[7] = bf16_hi(wu.w);
      }
      if (kr_f32) {
        float4* dst = reinterpret_cast<float4*>(kr_f32 + (dst0 + kr_row) * IRM_D_ROPE + (lane & 7) * 8);
        dst[0] = make_float4(f[0], f[1], f[2], f[3]);
        dst[1] = make_float4(f[4], f[5], f[6], f[7]);
      }
      __builtin_nontemporal_store(w, O + (dst0 + kr_row) * kUnitsPerRow + kLatUnits + (lane & 7));
    }
  }
}

}  // namespace

irm_status launch_prepare(const irm_table* t, const double* inv_freq, hipStream_t s) {
  InvFreq f;
  for (int i = 0; i < (int)kPairs; ++i) f.w[i] = inv_freq[i];
  const uint32_t map_blocks = (uint32_t)(((uint64_t)t->total_rows + kTile + 255) / 256);
  const uint32_t trig_blocks = (t->n_chunks * kPairs + 255) / 256;
  const uint32_t group_blocks = (t->n_groups + 255) / 256;
  const Image im = image_of(t);
  hipLaunchKernelGGL(prepare_kernel, dim3(map_blocks + trig_blocks + group_blocks), dim3(256), 0, s, im,
                     (uint32_t)t->total_rows, map_blocks, trig_blocks, t->n_groups, f, const_cast<uint4*>(im.rowmap),
                     const_cast<float2*>(im.trig), const_cast<uint4*>(im.items));
  return launch_check("table prepare kernel");
}

irm_status launch_trig(const irm_table* t, const double* inv_freq, hipStream_t s) {
  if (!t->n_chunks) return IRM_OK;
  InvFreq f;
  for (int i = 0; i < (int)kPairs; ++i) f.w[i] = inv_freq[i];
  const uint32_t n = t->n_chunks * kPairs;
  const Image im = image_of(t);
  hipLaunchKernelGGL(trig_kernel, dim3((n + 255) / 256), dim3(256), 0, s, im.ents, t->n_chunks, f,
                     const_cast<float2*>(im.trig));
  return launch_check("trig kernel");
}

irm_status launch_gather_index(const irm_table* t, int64_t* pool_row, int32_t* delta, hipStream_t s) {
  const uint32_t n = (uint32_t)t->total_rows;
  hipLaunchKernelGGL(gather_index_kernel, dim3((n + 255) / 256), dim3(256), 0, s, image_of(t), n, pool_row,
                     delta);
  return launch_check("gather index kernel");
}

irm_status launch_rotate_gather(const irm_table* t, const void* pool, void* out_kv, float* kr_f32,
                                hipStream_t s) {
  if (t->n_items == 0) return IRM_OK;  // no rows to assemble
  // one item per workgroup: at most total_rows / 8 + n_chunks items, below 2^31
  if (t->n_items > 0x7fffffffull) return fail(IRM_EUNSUPPORTED, "irm_rotate_gather: too many work items");
  hipLaunchKernelGGL(rotate_gather_kernel, dim3((uint32_t)t->n_items), dim3(kGatherThreads), 0, s, image_of(t),
                     static_cast<const uint4*>(pool), static_cast<uint4*>(out_kv), kr_f32,
                     pool_last_of(t->pool_rows));
  return launch_check("rotate-gather kernel");
}

}  // namespace irm
