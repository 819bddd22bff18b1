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
// table prepare, both passes in one launch.  Row map: one 16-byte record
// per assembled row, {pool row, delta (0 if fresh), entry (kNoRot if delta
// is 0), 0}, followed by kTile records of {0, 0, kNoRot, 0} so that
// whole-tile reads never leave the array; the first map_blocks workgroups
// write it (one row per thread), the rest the trig rows as trig_kernel does
// (one launch instead of two: 11.8 us against 13.4 us for the 64 x
// 32768-token batch; four rows per thread with one entry lookup took 25 us)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prepare_kernel(Image im, uint32_t total_rows, uint32_t map_blocks, InvFreq f,
                                                      uint4* __restrict__ rowmap, float2* __restrict__ trig) {
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
  const uint32_t idx = (blockIdx.x - map_blocks) * 256 + threadIdx.x;
  if (idx >= im.n_entries * irm::kPairs) return;
  const uint32_t e = idx / irm::kPairs, i = idx % irm::kPairs;
  const double phi = (double)im.ents[e].delta * f.w[i];
  double sn, cn;
  sincos(phi, &sn, &cn);
  trig[idx] = make_float2((float)cn, (float)sn);
}

// ---------------------------------------------------------------------------
// rotate-gather: a grid-stride stream over the assembled rows' 16-byte units
//
// Unit u is unit u % 72 of assembled row u / 72.  A workgroup is one wave;
// each lane keeps kUnitsInFlight units in flight per step, 64 apart, so the
// wave moves 1 KB per load and store instruction and a workgroup 4 KB; the
// row's record in the row map (pool row, entry) comes through the cache,
// shared by the 72 units of a row.  c_KV units are copied; k_r units of
// rotated rows are turned with the entry's (cos, sin).  Measured on the
// 64 x 32768-token batch: one-wave workgroups of 4 units per lane move
// 6.0-6.4 TB/s against 5.7 TB/s for four-wave workgroups (2-8 units per
// lane and 128-lane workgroups measured too), and with them pool loads
// through the cache beat non-temporal ones by 3-6%, behind a cache scrub as
// well as back to back; the stores stay non-temporal (plain stores: 5.7
// TB/s).  Short workgroups keep the chip's requests on a narrow window of
// addresses, as a plain copy of the same bytes shows (6.7 TB/s with one-wave
// workgroups, 5.9 TB/s with four-wave ones).
// ---------------------------------------------------------------------------
constexpr int kUnitsInFlight = 4;
constexpr int kGatherThreads = 64;
constexpr int kGatherStep = kUnitsInFlight * kGatherThreads;  // units per workgroup step

__global__ __launch_bounds__(kGatherThreads) void rotate_gather_kernel(Image im, uint64_t n_units,
                                                                  const uint4* __restrict__ pool,
                                                                  uint4* __restrict__ out,
                                                                  float* __restrict__ kr_f32) {
  const u32x4_t* P = reinterpret_cast<const u32x4_t*>(pool);
  u32x4_t* O = reinterpret_cast<u32x4_t*>(out);
  for (uint64_t base = (uint64_t)blockIdx.x * kGatherStep; base < n_units;
       base += (uint64_t)gridDim.x * kGatherStep) {
    uint64_t row[kUnitsInFlight];
    uint32_t col[kUnitsInFlight];
    uint4 rec[kUnitsInFlight];
#pragma unroll
    for (int k = 0; k < kUnitsInFlight; ++k) {
      const uint64_t u = min(base + (uint64_t)k * kGatherThreads + threadIdx.x, n_units - 1);
      row[k] = u / kUnitsPerRow;
      col[k] = (uint32_t)(u - row[k] * kUnitsPerRow);
      rec[k] = im.rowmap[row[k]];
    }
    u32x4_t v[kUnitsInFlight];
#pragma unroll
    for (int k = 0; k < kUnitsInFlight; ++k)
      v[k] = P[(size_t)rec[k].x * kUnitsPerRow + col[k]];
#pragma unroll
    for (int k = 0; k < kUnitsInFlight; ++k) {
      const uint64_t u = base + (uint64_t)k * kGatherThreads + threadIdx.x;
      if (u >= n_units) continue;
      u32x4_t w = v[k];
      if (col[k] >= (uint32_t)kLatUnits) {
        const uint32_t e = rec[k].z;
        float f[8];
        const uint4 wu = __builtin_bit_cast(uint4, w);
        if (e != kNoRot) {
          rotate_unit_f32(wu, im.trig + (size_t)e * kPairs + (col[k] - kLatUnits) * 4, f);
          w = u32x4_t{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])};
        } else {
          f[0] = bf16_lo(wu.x); f[1] = bf16_hi(wu.x); f[2] = bf16_lo(wu.y); f[3] = bf16_hi(wu.y);
          f[4] = bf16_lo(wu.z); f[5] = bf16_hi(wu.z); f[6] = bf16_lo(wu.w); f[7] = bf16_hi(wu.w);
        }
        if (kr_f32) {
          float4* dst = reinterpret_cast<float4*>(kr_f32 + row[k] * IRM_D_ROPE + (col[k] - kLatUnits) * 8);
          dst[0] = make_float4(f[0], f[1], f[2], f[3]);
          dst[1] = make_float4(f[4], f[5], f[6], f[7]);
        }
      }
      __builtin_nontemporal_store(w, O + u);
    }
  }
}

}  // namespace

irm_status launch_prepare(const irm_table* t, const double* inv_freq, hipStream_t s) {
  InvFreq f;
  for (int i = 0; i < (int)kPairs; ++i) f.w[i] = inv_freq[i];
  const uint32_t map_blocks = (uint32_t)(((uint64_t)t->total_rows + kTile + 255) / 256);
  const uint32_t trig_blocks = (t->n_chunks * kPairs + 255) / 256;
  const Image im = image_of(t);
  hipLaunchKernelGGL(prepare_kernel, dim3(map_blocks + trig_blocks), dim3(256), 0, s, im, (uint32_t)t->total_rows,
                     map_blocks, f, const_cast<uint4*>(im.rowmap), const_cast<float2*>(im.trig));
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
  const uint64_t n_units = t->total_rows * kUnitsPerRow;
  const uint64_t steps = (n_units + kGatherStep - 1) / kGatherStep;
  // one step per workgroup (measured faster than a persistent grid); the
  // grid-stride loop only covers grids past the launch limit
  const uint32_t grid = (uint32_t)(steps < 0x7fffffffull ? steps : 0x7fffffffull);
  hipLaunchKernelGGL(rotate_gather_kernel, dim3(grid), dim3(kGatherThreads), 0, s, image_of(t), n_units,
                     static_cast<const uint4*>(pool), static_cast<uint4*>(out_kv), kr_f32);
  return launch_check("rotate-gather kernel");
}

}  // namespace irm
