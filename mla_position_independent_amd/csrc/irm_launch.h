// Host-side launchers of the HIP kernels, one per kernel family.  Callers
// (the C ABI) validate every argument first; a launcher only shapes the grid
// and reports launch errors.
#pragma once

#include <hip/hip_runtime.h>

#include "irm_internal.h"

namespace irm {

irm_status hip_check(hipError_t err, const char* what);
irm_status launch_check(const char* what);

// irm_gather.hip
irm_status launch_trig(const irm_table* t, const double* inv_freq, hipStream_t s);
irm_status launch_prepare(const irm_table* t, const double* inv_freq, hipStream_t s);  // row map + trig, one launch
irm_status launch_gather_index(const irm_table* t, int64_t* pool_row, int32_t* delta, hipStream_t s);
irm_status launch_rotate_gather(const irm_table* t, const void* pool, void* out_kv, float* kr_f32,
                                hipStream_t s);

// irm_decode.hip: split count used when the caller passes 0, and the launch
// of both decode passes into a workspace laid out as [acc | ml].
uint32_t decode_default_splits(const irm_table* t, uint32_t n_groups);
// Partial states per sequence the split pass writes for n_splits splits (the
// 64-head kernel merges runs of splits when the device has fewer compute
// units than (sequence, split, head block) triples).
uint32_t decode_parts(const irm_table* t, uint32_t n_heads, uint32_t n_splits);
// The library's own decode workspace for callers that cannot allocate: a
// device array of kDecodeScratchBytes per device, its address looked up
// once per device (hipGetSymbolAddress) with that device current.
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
irm_status decode_scratch(void** ptr);
irm_status launch_decode(const irm_table* t, const void* q_lat, const void* q_rope, const void* pool,
                         uint64_t pool_rows, uint32_t n_heads, uint32_t n_splits, float scale, void* out,
                         float* lse, float* ws_acc, float* ws_ml, hipStream_t s);

// irm_prefill.hip
irm_status launch_prefill(const irm_table* t, const void* q_lat, const void* q_rope, int32_t q_pos0,
                          uint32_t n_q, const void* pool, uint64_t pool_rows, uint32_t n_heads, float scale,
                          void* out, float* lse, hipStream_t s);
constexpr uint32_t kGqaMaxHeadDim = 256;
irm_status launch_gqa_rotate_gather(const irm_table* t, const void* pool, uint32_t n_kv_heads, uint32_t head_dim,
                                    const double* inv_freq, float2* trig, void* out, hipStream_t s);
irm_status launch_prefill_assembled(const void* q_lat, const void* q_rope, int32_t q_pos0, uint32_t n_q,
                                    const void* kv, uint64_t kv_rows, uint32_t n_heads, float scale, void* out,
                                    float* lse, hipStream_t s);

// irm_nonabsorbed.hip
irm_status launch_kv_upproj(const void* kv, uint64_t kv_rows, const void* w_uk, const void* w_uv, uint32_t n_heads,
                            void* out, hipStream_t s);
irm_status launch_prefill_nonabsorbed(const void* q_nope, const void* q_rope, int32_t q_pos0, uint32_t n_q,
                                      const void* kv, const void* kvh, uint64_t kv_rows, uint32_t n_heads,
                                      float scale, void* out, float* lse, hipStream_t s);

// Last pool row a kernel may touch (pool_rows is clamped to 2^32).
inline uint32_t pool_last_of(uint64_t pool_rows) {
  return (uint32_t)((pool_rows < 0x100000000ull ? pool_rows : 0x100000000ull) - 1);
}

}  // namespace irm
