// C ABI entry points: argument validation, then the kernel launchers.
//
// The operations follow the Irminsul pages (arXiv:2605.05696); each entry
// point's declaration in irm.h cites the passage that defines it.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <string>

#include "irm_internal.h"
#include "irm_launch.h"

using irm::fail;

namespace irm {

irm_status hip_check(hipError_t err, const char* what) {
  if (err == hipSuccess) return IRM_OK;
  return fail(IRM_EHIP, std::string(what) + ": " + hipGetErrorString(err));
}

irm_status launch_check(const char* what) { return hip_check(hipGetLastError(), what); }

}  // namespace irm

namespace {

using irm::hip_check;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The kernels are built for gfx950 only; refuse other devices up front.
irm_status check_device() {
  static thread_local int checked_dev = -1;
  int dev = 0;
  irm_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (st != IRM_OK) return st;
  if (dev == checked_dev) return IRM_OK;
  hipDeviceProp_t prop;
  st = hip_check(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties");
  if (st != IRM_OK) return st;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(IRM_EUNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", kernels are built for gfx950");
  checked_dev = dev;
  return IRM_OK;
}

irm_status need_uploaded(const irm_table* t, const char* fn) {
  if (!t) return fail(IRM_EINVAL, std::string(fn) + ": table is NULL");
  if (!t->dev) return fail(IRM_EINVAL, std::string(fn) + ": table has not been uploaded");
  return IRM_OK;
}

irm_status check_pool(const irm_table* t, const void* pool, uint64_t pool_rows, const char* fn) {
  if (t->n_chunks && !pool) return fail(IRM_EINVAL, std::string(fn) + ": pool is NULL");
  if (!aligned16(pool)) return fail(IRM_EINVAL, std::string(fn) + ": pool must be 16-byte aligned");
  if (pool_rows < t->pool_rows)
    return fail(IRM_ERANGE, std::string(fn) + ": pool has fewer rows than the table was built for");
  return IRM_OK;
}

irm_status check_heads(uint32_t n_heads, const char* fn) {
  if (n_heads == 0 || n_heads % 16 != 0 || n_heads > IRM_MAX_HEADS)
    return fail(IRM_EUNSUPPORTED, std::string(fn) + ": n_heads must be a multiple of 16, at most 128");
  return IRM_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" irm_status irm_table_upload(irm_table* t, const double* inv_freq, void* dev_buf,
                                       size_t dev_bytes, void* stream) {
  if (!t) return fail(IRM_EINVAL, "irm_table_upload: table is NULL");
  if (!inv_freq) return fail(IRM_EINVAL, "irm_table_upload: inv_freq is NULL");
  if (!dev_buf) return fail(IRM_EINVAL, "irm_table_upload: dev_buf is NULL");
  if (reinterpret_cast<uintptr_t>(dev_buf) % irm::kAlign)
    return fail(IRM_EINVAL, "irm_table_upload: dev_buf must be 256-byte aligned");
  if (dev_bytes < t->layout.bytes)
    return fail(IRM_EWORKSPACE, "irm_table_upload: dev_buf smaller than the device image");
  for (int i = 0; i < (int)irm::kPairs; ++i)
    if (!std::isfinite(inv_freq[i])) return fail(IRM_EINVAL, "irm_table_upload: inv_freq not finite");
  irm_status st = check_device();
  if (st != IRM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_check(hipMemcpyAsync(dev_buf, t->image.data(), t->layout.off_trig, hipMemcpyHostToDevice, s),
                 "irm_table_upload: hipMemcpyAsync");
  if (st != IRM_OK) return st;
  t->dev = dev_buf;
  st = irm_table_prepare(t, inv_freq, stream);
  if (st != IRM_OK) t->dev = nullptr;
  return st;
}

extern "C" irm_status irm_table_prepare(irm_table* t, const double* inv_freq, void* stream) {
  irm_status st = need_uploaded(t, "irm_table_prepare");
  if (st != IRM_OK) return st;
  if (!inv_freq) return fail(IRM_EINVAL, "irm_table_prepare: inv_freq is NULL");
  for (int i = 0; i < (int)irm::kPairs; ++i)
    if (!std::isfinite(inv_freq[i])) return fail(IRM_EINVAL, "irm_table_prepare: inv_freq not finite");
  if ((st = check_device()) != IRM_OK) return st;
  std::memcpy(t->inv_freq, inv_freq, sizeof(t->inv_freq));
  return irm::launch_prepare(t, inv_freq, static_cast<hipStream_t>(stream));
}

extern "C" irm_status irm_table_set_rope(irm_table* t, const double* inv_freq, void* stream) {
  irm_status st = need_uploaded(t, "irm_table_set_rope");
  if (st != IRM_OK) return st;
  if (!inv_freq) return fail(IRM_EINVAL, "irm_table_set_rope: inv_freq is NULL");
  for (int i = 0; i < (int)irm::kPairs; ++i)
    if (!std::isfinite(inv_freq[i])) return fail(IRM_EINVAL, "irm_table_set_rope: inv_freq not finite");
  if (!t->n_chunks) return IRM_OK;
  std::memcpy(t->inv_freq, inv_freq, sizeof(t->inv_freq));
  return irm::launch_trig(t, inv_freq, static_cast<hipStream_t>(stream));
}

extern "C" irm_status irm_table_gather_index(const irm_table* t, int64_t* pool_row, int32_t* delta,
                                             void* stream) {
  irm_status st = need_uploaded(t, "irm_table_gather_index");
  if (st != IRM_OK) return st;
  if (t->total_rows == 0 || (!pool_row && !delta)) return IRM_OK;
  return irm::launch_gather_index(t, pool_row, delta, static_cast<hipStream_t>(stream));
}

extern "C" irm_status irm_rotate_gather(const irm_table* t, const void* pool, uint64_t pool_rows,
                                        void* out_kv, float* kr_f32, void* stream) {
  irm_status st = need_uploaded(t, "irm_rotate_gather");
  if (st != IRM_OK) return st;
  if (t->total_rows == 0) return IRM_OK;
  if ((st = check_pool(t, pool, pool_rows, "irm_rotate_gather")) != IRM_OK) return st;
  if (!out_kv || !aligned16(out_kv)) return fail(IRM_EINVAL, "irm_rotate_gather: out_kv NULL or misaligned");
  if (kr_f32 && !aligned16(kr_f32)) return fail(IRM_EINVAL, "irm_rotate_gather: kr_f32 misaligned");
  return irm::launch_rotate_gather(t, pool, out_kv, kr_f32, static_cast<hipStream_t>(stream));
}

extern "C" irm_status irm_mla_decode_workspace(const irm_table* t, uint32_t n_heads, uint32_t n_splits,
                                               size_t* bytes) {
  if (!t || !bytes) return fail(IRM_EINVAL, "irm_mla_decode_workspace: NULL argument");
  irm_status st = check_heads(n_heads, "irm_mla_decode_workspace");
  if (st != IRM_OK) return st;
  const uint32_t S = n_splits ? n_splits : irm::decode_default_splits(t, n_heads / 16);
  const size_t parts = (size_t)t->n_seq * S * n_heads;
  *bytes = irm::align_up(parts * IRM_D_LATENT * sizeof(float)) + irm::align_up(parts * 2 * sizeof(float));
  return IRM_OK;
}

extern "C" irm_status irm_mla_decode(const void* q_latent, const void* q_rope, const irm_table* t,
                                     const void* pool, uint64_t pool_rows, uint32_t n_heads,
                                     uint32_t n_splits, float scale, void* out, float* lse,
                                     void* workspace, size_t ws_bytes, void* stream) {
  irm_status st = need_uploaded(t, "irm_mla_decode");
  if (st != IRM_OK) return st;
  if ((st = check_heads(n_heads, "irm_mla_decode")) != IRM_OK) return st;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(IRM_EINVAL, "irm_mla_decode: scale must be finite and > 0");
  if (t->n_seq == 0) return IRM_OK;
  if (t->min_seq_len == 0) return fail(IRM_EINVAL, "irm_mla_decode: every sequence needs at least one row");
  if ((st = check_pool(t, pool, pool_rows, "irm_mla_decode")) != IRM_OK) return st;
  if (!q_latent || !q_rope || !out || !aligned16(q_latent) || !aligned16(q_rope) || !aligned16(out))
    return fail(IRM_EINVAL, "irm_mla_decode: q_latent, q_rope and out must be non-NULL and 16-byte aligned");
  if (n_splits > 4096) return fail(IRM_EUNSUPPORTED, "irm_mla_decode: n_splits above 4096");
  const uint32_t G = n_heads / 16;
  const uint32_t S = n_splits ? n_splits : irm::decode_default_splits(t, G);
  size_t need = 0;
  irm_mla_decode_workspace(t, n_heads, S, &need);
  if (!workspace || ws_bytes < need || reinterpret_cast<uintptr_t>(workspace) % irm::kAlign)
    return fail(IRM_EWORKSPACE, "irm_mla_decode: workspace missing, misaligned or smaller than "
                                "irm_mla_decode_workspace");
  const size_t parts = (size_t)t->n_seq * S * n_heads;
  if ((st = check_device()) != IRM_OK) return st;
  float* ws_acc = static_cast<float*>(workspace);
  float* ws_ml = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) +
                                          irm::align_up(parts * IRM_D_LATENT * sizeof(float)));
  return irm::launch_decode(t, q_latent, q_rope, pool, pool_rows, n_heads, S, scale, out, lse, ws_acc, ws_ml,
                            static_cast<hipStream_t>(stream));
}

extern "C" irm_status irm_mla_decode_noalloc(const void* q_latent, const void* q_rope, const irm_table* t,
                                             const void* pool, uint64_t pool_rows, uint32_t n_heads,
                                             uint32_t n_splits, float scale, void* out, float* lse, void* stream) {
  static const char* fn = "irm_mla_decode_noalloc";
  irm_status st = need_uploaded(t, fn);
  if (st != IRM_OK) return st;
  if ((st = check_heads(n_heads, fn)) != IRM_OK) return st;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(IRM_EINVAL, std::string(fn) + ": scale must be finite and > 0");
  if (t->n_seq == 0) return IRM_OK;
  if (t->min_seq_len == 0) return fail(IRM_EINVAL, std::string(fn) + ": every sequence needs at least one row");
  if ((st = check_pool(t, pool, pool_rows, fn)) != IRM_OK) return st;
  if (!q_latent || !q_rope || !out || !aligned16(q_latent) || !aligned16(q_rope) || !aligned16(out))
    return fail(IRM_EINVAL, std::string(fn) + ": q_latent, q_rope and out must be non-NULL and 16-byte aligned");
  if (n_splits > 4096) return fail(IRM_EUNSUPPORTED, std::string(fn) + ": n_splits above 4096");
  if ((st = check_device()) != IRM_OK) return st;
  const uint32_t S = n_splits ? n_splits : irm::decode_default_splits(t, n_heads / 16);
  // the split pass writes n_parts partial states per (sequence, head)
  const size_t parts = (size_t)t->n_seq * irm::decode_parts(t, n_heads, S) * n_heads;
  const size_t acc_bytes = irm::align_up(parts * IRM_D_LATENT * sizeof(float));
  const size_t need = acc_bytes + irm::align_up(parts * 2 * sizeof(float));
  if (need > irm::kDecodeScratchBytes)
    return fail(IRM_EWORKSPACE, std::string(fn) + ": partial states need " + std::to_string(need) +
                                    " bytes, more than the library's " + std::to_string(irm::kDecodeScratchBytes) +
                                    "-byte scratch; use irm_mla_decode with a caller workspace");
  void* ws = nullptr;
  if ((st = irm::decode_scratch(&ws)) != IRM_OK) return st;
  float* ws_acc = static_cast<float*>(ws);
  float* ws_ml = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + acc_bytes);
  return irm::launch_decode(t, q_latent, q_rope, pool, pool_rows, n_heads, S, scale, out, lse, ws_acc, ws_ml,
                            static_cast<hipStream_t>(stream));
}

extern "C" irm_status irm_mla_prefill_tail(const void* q_latent, const void* q_rope, int32_t q_pos0,
                                           uint32_t n_q, const irm_table* t, const void* pool,
                                           uint64_t pool_rows, uint32_t n_heads, float scale,
                                           void* out, float* lse, void* stream) {
  irm_status st = need_uploaded(t, "irm_mla_prefill_tail");
  if (st != IRM_OK) return st;
  if ((st = check_heads(n_heads, "irm_mla_prefill_tail")) != IRM_OK) return st;
  if (t->n_seq != 1) return fail(IRM_EINVAL, "irm_mla_prefill_tail: table must hold exactly one sequence");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(IRM_EINVAL, "irm_mla_prefill_tail: scale must be finite and > 0");
  if (q_pos0 < 0 || n_q == 0 || (uint64_t)q_pos0 + n_q > t->total_rows)
    return fail(IRM_ERANGE, "irm_mla_prefill_tail: queries must satisfy 0 <= q_pos0, 1 <= n_q, q_pos0 + n_q <= N");
  if ((st = check_pool(t, pool, pool_rows, "irm_mla_prefill_tail")) != IRM_OK) return st;
  if (!q_latent || !q_rope || !out || !aligned16(q_latent) || !aligned16(q_rope) || !aligned16(out))
    return fail(IRM_EINVAL, "irm_mla_prefill_tail: q_latent, q_rope and out must be non-NULL and 16-byte aligned");
  if ((st = check_device()) != IRM_OK) return st;
  return irm::launch_prefill(t, q_latent, q_rope, q_pos0, n_q, pool, pool_rows, n_heads, scale, out, lse,
                             static_cast<hipStream_t>(stream));
}

extern "C" irm_status irm_mla_prefill_assembled(const void* q_latent, const void* q_rope, int32_t q_pos0,
                                                uint32_t n_q, const void* kv, uint64_t kv_rows, uint32_t n_heads,
                                                float scale, void* out, float* lse, void* stream) {
  static const char* fn = "irm_mla_prefill_assembled";
  irm_status st = check_heads(n_heads, fn);
  if (st != IRM_OK) return st;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(IRM_EINVAL, std::string(fn) + ": scale must be finite and > 0");
  if (kv_rows > 0x100000000ull) return fail(IRM_EUNSUPPORTED, std::string(fn) + ": at most 2^32 cache rows");
  if (q_pos0 < 0 || n_q == 0 || (uint64_t)q_pos0 + n_q > kv_rows)
    return fail(IRM_ERANGE, std::string(fn) + ": queries must satisfy 0 <= q_pos0, 1 <= n_q, q_pos0 + n_q <= kv_rows");
  if (!kv || !aligned16(kv)) return fail(IRM_EINVAL, std::string(fn) + ": kv must be non-NULL and 16-byte aligned");
  if (!q_latent || !q_rope || !out || !aligned16(q_latent) || !aligned16(q_rope) || !aligned16(out))
    return fail(IRM_EINVAL, std::string(fn) + ": q_latent, q_rope and out must be non-NULL and 16-byte aligned");
  if ((st = check_device()) != IRM_OK) return st;
  return irm::launch_prefill_assembled(q_latent, q_rope, q_pos0, n_q, kv, kv_rows, n_heads, scale, out, lse,
                                       static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// Non-absorbed prefill
// ---------------------------------------------------------------------------
namespace {
irm_status check_na_shape(uint64_t kv_rows, uint32_t n_heads, const char* fn) {
  if (n_heads < 1 || n_heads > 128) return fail(IRM_EUNSUPPORTED, std::string(fn) + ": n_heads must be in [1, 128]");
  if (kv_rows >= 0x100000000ull) return fail(IRM_EUNSUPPORTED, std::string(fn) + ": fewer than 2^32 cache rows");
  return IRM_OK;
}
}  // namespace

extern "C" irm_status irm_mla_kv_upproj(const void* kv, uint64_t kv_rows, const void* w_uk, const void* w_uv,
                                        uint32_t n_heads, void* out, void* stream) {
  static const char* fn = "irm_mla_kv_upproj";
  irm_status st = check_na_shape(kv_rows, n_heads, fn);
  if (st != IRM_OK) return st;
  if (kv_rows && (!kv || !w_uk || !w_uv || !out || !aligned16(kv) || !aligned16(w_uk) || !aligned16(w_uv) ||
                  !aligned16(out)))
    return fail(IRM_EINVAL, std::string(fn) + ": kv, w_uk, w_uv and out must be non-NULL and 16-byte aligned");
  if ((st = check_device()) != IRM_OK) return st;
  return irm::launch_kv_upproj(kv, kv_rows, w_uk, w_uv, n_heads, out, static_cast<hipStream_t>(stream));
}

extern "C" irm_status irm_mla_prefill_nonabsorbed(const void* q_nope, const void* q_rope, int32_t q_pos0,
                                                  uint32_t n_q, const void* kv, const void* kvh, uint64_t kv_rows,
                                                  uint32_t n_heads, float scale, void* out, float* lse,
                                                  void* stream) {
  static const char* fn = "irm_mla_prefill_nonabsorbed";
  irm_status st = check_na_shape(kv_rows, n_heads, fn);
  if (st != IRM_OK) return st;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(IRM_EINVAL, std::string(fn) + ": scale must be finite and > 0");
  if (q_pos0 < 0 || n_q == 0 || (uint64_t)q_pos0 + n_q > kv_rows)
    return fail(IRM_ERANGE, std::string(fn) + ": queries must satisfy 0 <= q_pos0, 1 <= n_q, q_pos0 + n_q <= kv_rows");
  if (!kv || !kvh || !aligned16(kv) || !aligned16(kvh))
    return fail(IRM_EINVAL, std::string(fn) + ": kv and kvh must be non-NULL and 16-byte aligned");
  if (!q_nope || !q_rope || !out || !aligned16(q_nope) || !aligned16(q_rope) || !aligned16(out))
    return fail(IRM_EINVAL, std::string(fn) + ": q_nope, q_rope and out must be non-NULL and 16-byte aligned");
  if ((st = check_device()) != IRM_OK) return st;
  return irm::launch_prefill_nonabsorbed(q_nope, q_rope, q_pos0, n_q, kv, kvh, kv_rows, n_heads, scale, out, lse,
                                         static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// GQA/MHA comparison path
// ---------------------------------------------------------------------------
namespace {
irm_status check_gqa_shape(uint32_t n_kv_heads, uint32_t head_dim, const char* fn) {
  if (head_dim < 16 || head_dim > irm::kGqaMaxHeadDim || head_dim % 16)
    return fail(IRM_EUNSUPPORTED, std::string(fn) + ": head_dim must be a multiple of 16 in [16, 256]");
  if (n_kv_heads < 1 || n_kv_heads > 256)
    return fail(IRM_EUNSUPPORTED, std::string(fn) + ": n_kv_heads must be in [1, 256]");
  return IRM_OK;
}
}  // namespace

extern "C" irm_status irm_gqa_workspace(const irm_table* t, uint32_t head_dim, size_t* bytes) {
  if (!t || !bytes) return fail(IRM_EINVAL, "irm_gqa_workspace: NULL argument");
  irm_status st = check_gqa_shape(1, head_dim, "irm_gqa_workspace");
  if (st != IRM_OK) return st;
  *bytes = (size_t)t->n_chunks * (head_dim / 2) * 8;
  return IRM_OK;
}

extern "C" irm_status irm_gqa_rotate_gather(const irm_table* t, const void* pool, uint64_t pool_rows,
                                            uint32_t n_kv_heads, uint32_t head_dim, const double* inv_freq,
                                            void* ws, size_t ws_bytes, void* out, void* stream) {
  static const char* fn = "irm_gqa_rotate_gather";
  irm_status st = need_uploaded(t, fn);
  if (st != IRM_OK) return st;
  if ((st = check_gqa_shape(n_kv_heads, head_dim, fn)) != IRM_OK) return st;
  if (!inv_freq) return fail(IRM_EINVAL, std::string(fn) + ": inv_freq is NULL");
  for (uint32_t i = 0; i < head_dim / 2; ++i)
    if (!std::isfinite(inv_freq[i])) return fail(IRM_EINVAL, std::string(fn) + ": inv_freq must be finite");
  if ((st = check_pool(t, pool, pool_rows, fn)) != IRM_OK) return st;
  const size_t need = (size_t)t->n_chunks * (head_dim / 2) * 8;
  if (need && (!ws || ws_bytes < need || !aligned16(ws)))
    return fail(IRM_EWORKSPACE, std::string(fn) + ": workspace missing, unaligned or smaller than irm_gqa_workspace");
  if (t->total_rows && (!out || !aligned16(out)))
    return fail(IRM_EINVAL, std::string(fn) + ": out must be non-NULL and 16-byte aligned");
  if ((st = check_device()) != IRM_OK) return st;
  return irm::launch_gqa_rotate_gather(t, pool, n_kv_heads, head_dim, inv_freq, static_cast<float2*>(ws), out,
                                       static_cast<hipStream_t>(stream));
}

