// GQA/MHA comparison path: position-independent reuse of a grouped-query KV
// cache, where every reused row must have the whole key of every KV head
// rotated (the correction of earlier position-independent caching systems,
// O(N d_K) per KV head, against MLA's 64-wide k_r slice: gist.science
// summary, section 1; gentlecold.top article, sections 3 and 4).  The same
// chunk table, row map and per-entry delta as the MLA rotate-gather.
//
// Row layout: [K of n_kv_heads heads | V of n_kv_heads heads], head_dim bf16
// per head.  The rotation covers the whole head_dim with the half-split
// pairing of GQA models: element i turns with element i + head_dim/2 by the
// angle delta * omega_i.

#include <hip/hip_runtime.h>

#include "irm_device.h"
#include "irm_launch.h"

namespace irm {
namespace {

using namespace irm::dev;

struct GqaFreq {
  double w[kGqaMaxHeadDim / 2];
};

// cos/sin(delta_e * omega_i) in double, stored float2: [n_entries][head_dim/2]
__global__ void gqa_trig_kernel(const DevEntry* __restrict__ ents, uint32_t n_entries, uint32_t half, GqaFreq f,
                                float2* __restrict__ trig) {
  const uint64_t idx = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (uint64_t)n_entries * half) return;
  const uint32_t e = (uint32_t)(idx / half), i = (uint32_t)(idx % half);
  double s, c;
  sincos((double)ents[e].delta * f.w[i], &s, &c);
  trig[idx] = make_float2((float)c, (float)s);
}

// A grid-stride stream over items of the assembled rows: per row first the
// K pairs (unit j of a head's first half with unit j of its second half, 32
// bytes: the two halves of 8 rotation pairs), then the V units (16 bytes).
// Pair units of rows with a nonzero delta are turned in float with the
// entry's (cos, sin) and rounded to bf16 (RNE); everything else is copied.
// A workgroup is one wave with one item per lane, pool loads through the
// cache and non-temporal stores: on the 64 x 32768-token batch over an
// 8 x 128 pool this moves 6.4 TB/s, against 5.4 TB/s for four-wave
// workgroups of four items per lane with non-temporal loads (2-4 items per
// lane and 128-256-lane workgroups measured between the two).
constexpr int kItemsInFlight = 1;
constexpr int kGqaThreads = 64;
constexpr int kGqaStep = kItemsInFlight * kGqaThreads;

struct GqaShape {
  uint32_t half_units;  // units in half a head (head_dim / 16)
  uint32_t head_units;  // units per head (head_dim / 8)
  uint32_t n_pairs;     // K pair items per row (n_kv_heads * head_dim / 16)
  uint32_t row_units;   // units per row (n_kv_heads * head_dim / 4)
  uint32_t items;       // items per row (n_pairs + n_kv_heads * head_dim / 8)
  uint32_t half;        // rotation pairs per head (head_dim / 2)
  uint64_t recip;       // ceil(2^64 / items): item / items == umulhi(item, recip) for item < 2^64 / items
};

__device__ __forceinline__ u32x4_t turn(const u32x4_t& a, const u32x4_t& b, const float2* cs, bool hi) {
  // a holds x_i, b holds x_{i+h} for 8 consecutive i; returns the new a (hi = false) or b (hi = true)
  u32x4_t r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float2 c0 = cs[2 * q], c1 = cs[2 * q + 1];
    const float x0 = bf16_lo(a[q]), x1 = bf16_hi(a[q]), y0 = bf16_lo(b[q]), y1 = bf16_hi(b[q]);
    r[q] = hi ? pack_bf16(fmaf(x0, c0.y, y0 * c0.x), fmaf(x1, c1.y, y1 * c1.x))
              : pack_bf16(fmaf(x0, c0.x, -(y0 * c0.y)), fmaf(x1, c1.x, -(y1 * c1.y)));
  }
  return r;
}

__global__ __launch_bounds__(kGqaThreads) void gqa_rotate_gather_kernel(const uint4* __restrict__ rowmap,
                                                                      uint64_t n_items, GqaShape g,
                                                                      const float2* __restrict__ trig,
                                                                      const uint4* __restrict__ pool,
                                                                      uint4* __restrict__ out) {
  const u32x4_t* P = reinterpret_cast<const u32x4_t*>(pool);
  u32x4_t* O = reinterpret_cast<u32x4_t*>(out);
  for (uint64_t base = (uint64_t)blockIdx.x * kGqaStep; base < n_items; base += (uint64_t)gridDim.x * kGqaStep) {
    uint64_t row[kItemsInFlight];
    uint32_t col[kItemsInFlight];
    uint4 rec[kItemsInFlight];
#pragma unroll
    for (int k = 0; k < kItemsInFlight; ++k) {
      const uint64_t it = min(base + (uint64_t)k * kGqaThreads + threadIdx.x, n_items - 1);
      row[k] = __umul64hi(it, g.recip);
      col[k] = (uint32_t)(it - row[k] * g.items);
      rec[k] = rowmap[row[k]];
    }
    // source / destination units: a pair item reads two units, a V item one
    uint32_t u0[kItemsInFlight], u1[kItemsInFlight];
    u32x4_t a[kItemsInFlight], b[kItemsInFlight];
#pragma unroll
    for (int k = 0; k < kItemsInFlight; ++k) {
      if (col[k] < g.n_pairs) {
        const uint32_t h = col[k] / g.half_units, j = col[k] - h * g.half_units;
        u0[k] = h * g.head_units + j;
        u1[k] = u0[k] + g.half_units;
      } else {
        u0[k] = g.row_units / 2 + (col[k] - g.n_pairs);
        u1[k] = u0[k];
      }
      const u32x4_t* src = P + (size_t)rec[k].x * g.row_units;
      a[k] = src[u0[k]];
      b[k] = col[k] < g.n_pairs ? src[u1[k]] : a[k];
    }
#pragma unroll
    for (int k = 0; k < kItemsInFlight; ++k) {
      const uint64_t it = base + (uint64_t)k * kGqaThreads + threadIdx.x;
      if (it >= n_items) continue;
      u32x4_t* dst = O + (size_t)row[k] * g.row_units;
      if (col[k] < g.n_pairs) {
        u32x4_t lo = a[k], hi = b[k];
        if (rec[k].z != kNoRot) {
          const uint32_t j = col[k] % g.half_units;
          const float2* cs = trig + (size_t)rec[k].z * g.half + 8 * j;
          lo = turn(a[k], b[k], cs, false);
          hi = turn(a[k], b[k], cs, true);
        }
        __builtin_nontemporal_store(lo, dst + u0[k]);
        __builtin_nontemporal_store(hi, dst + u1[k]);
      } else {
        __builtin_nontemporal_store(a[k], dst + u0[k]);
      }
    }
  }
}

}  // namespace

irm_status launch_gqa_rotate_gather(const irm_table* t, const void* pool, uint32_t n_kv_heads, uint32_t head_dim,
                                    const double* inv_freq, float2* trig, void* out, hipStream_t s) {
  const Image im = image_of(t);
  const uint32_t half = head_dim / 2;
  if (t->n_chunks) {
    GqaFreq f{};
    for (uint32_t i = 0; i < half; ++i) f.w[i] = inv_freq[i];
    const uint64_t n = (uint64_t)t->n_chunks * half;
    hipLaunchKernelGGL(gqa_trig_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, s, im.ents, t->n_chunks,
                       half, f, trig);
    const irm_status st = launch_check("GQA trig kernel");
    if (st != IRM_OK) return st;
  }
  if (!t->total_rows) return IRM_OK;
  GqaShape g;
  g.half_units = head_dim / 16;
  g.head_units = head_dim / 8;
  g.n_pairs = n_kv_heads * head_dim / 16;
  g.row_units = n_kv_heads * head_dim / 4;
  g.items = g.n_pairs + n_kv_heads * head_dim / 8;
  g.half = half;
  // exact quotient by multiplication (Granlund and Montgomery, "Division by
  // invariant integers using multiplication", 1994): with recip = ceil(2^64 / d)
  // the error term stays below one for numerators under 2^64 / d; items <= 12288
  // and rows < 2^32 keep every item index far below that
  g.recip = (uint64_t)((((unsigned __int128)1 << 64) + g.items - 1) / g.items);
  const uint64_t n_items = t->total_rows * g.items;
  const uint64_t steps = (n_items + kGqaStep - 1) / kGqaStep;
  const uint32_t grid = (uint32_t)(steps < 0x7fffffffull ? steps : 0x7fffffffull);
  hipLaunchKernelGGL(gqa_rotate_gather_kernel, dim3(grid), dim3(kGqaThreads), 0, s, im.rowmap, n_items, g, trig,
                     static_cast<const uint4*>(pool), static_cast<uint4*>(out));
  return launch_check("GQA rotate-gather kernel");
}

}  // namespace irm
