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
// row map: one 16-byte record per assembled row, {pool row, delta (0 if
// fresh), entry (kNoRot if delta is 0), 0}, followed by kTile records of
// {0, 0, kNoRot, 0} so that whole-tile reads never leave the array
// ---------------------------------------------------------------------------
__global__ void rowmap_kernel(Image im, uint32_t total_rows, uint4* __restrict__ rowmap) {
  const uint32_t g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= total_rows + kTile) return;
  if (g >= total_rows) {
    rowmap[g] = make_uint4(0u, 0u, kNoRot, 0u);
    return;
  }
  const uint32_t e = find_entry(im, g);
  const DevEntry d = im.ents[e];
  rowmap[g] = make_uint4(d.pool_row + (g - d.out_row), (uint32_t)d.delta, d.delta != 0 ? e : kNoRot, 0u);
}

// ---------------------------------------------------------------------------
// rotate-gather: one workgroup per 64 assembled rows, flat 16-byte units
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void rotate_gather_kernel(Image im, uint32_t total_rows,
                                                                  const uint4* __restrict__ pool,
                                                                  uint4* __restrict__ out,
                                                                  float* __restrict__ kr_f32) {
  __shared__ uint32_t s_src[kTile];
  __shared__ uint32_t s_rot[kTile];
  const uint32_t tile0 = blockIdx.x * kTile;
  const int tid = threadIdx.x;
  const uint32_t nrows = min((uint32_t)kTile, total_rows - tile0);
  if (tid < kTile) {
    uint32_t src = 0, rot = kNoRot;
    if ((uint32_t)tid < nrows) {
      const uint32_t g = tile0 + tid;
      const uint32_t e = find_entry(im, g);
      const DevEntry d = im.ents[e];
      src = d.pool_row + (g - d.out_row);
      rot = d.delta != 0 ? e : kNoRot;
    }
    s_src[tid] = src;
    s_rot[tid] = rot;
  }
  __syncthreads();
  const uint32_t nunits = nrows * kUnitsPerRow;
  uint4 v[kUnitsPerThread];
#pragma unroll
  for (int k = 0; k < kUnitsPerThread; ++k) {
    const uint32_t u = tid + k * kThreads;
    if (u < nunits) {
      const uint32_t r = u / kUnitsPerRow, c = u - r * kUnitsPerRow;
      v[k] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                                            pool + (size_t)s_src[r] * kUnitsPerRow + c)));
    }
  }
#pragma unroll
  for (int k = 0; k < kUnitsPerThread; ++k) {
    const uint32_t u = tid + k * kThreads;
    if (u < nunits) {
      const uint32_t r = u / kUnitsPerRow, c = u - r * kUnitsPerRow;
      uint4 w = v[k];
      if (c >= (uint32_t)kLatUnits) {
        const uint32_t e = s_rot[r];
        float f[8];
        if (e != kNoRot) {
          rotate_unit_f32(w, im.trig + (size_t)e * irm::kPairs + (c - kLatUnits) * 4, f);
          w = make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]),
                         pack_bf16(f[6], f[7]));
        } else {
          f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
          f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
        }
        if (kr_f32) {
          float4* dst = reinterpret_cast<float4*>(kr_f32 + (size_t)(tile0 + r) * IRM_D_ROPE +
                                                  (c - kLatUnits) * 8);
          dst[0] = make_float4(f[0], f[1], f[2], f[3]);
          dst[1] = make_float4(f[4], f[5], f[6], f[7]);
        }
      }
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, w),
                                  reinterpret_cast<u32x4_t*>(out + (size_t)(tile0 + r) * kUnitsPerRow + c));
    }
  }
}

}  // namespace

irm_status launch_rowmap(const irm_table* t, hipStream_t s) {
  const uint32_t n = (uint32_t)t->total_rows;
  const Image im = image_of(t);
  hipLaunchKernelGGL(rowmap_kernel, dim3((n + kTile + 255) / 256), dim3(256), 0, s, im, n,
                     const_cast<uint4*>(im.rowmap));
  return launch_check("row map kernel");
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
  const uint32_t n = (uint32_t)t->total_rows;
  hipLaunchKernelGGL(rotate_gather_kernel, dim3((n + kTile - 1) / kTile), dim3(kThreads), 0, s, image_of(t), n,
                     static_cast<const uint4*>(pool), static_cast<uint4*>(out_kv), kr_f32);
  return launch_check("rotate-gather kernel");
}

}  // namespace irm
