// Chunked tail-prefill: causal absorbed MLA attention of a block of new
// query tokens over the assembled cache, with the delta rotation applied as
// KV rows are loaded (Irminsul pages: gentlecold.top article, sections 4, 5
// and 15; gist.science summary, section 2.2).

#include <hip/hip_runtime.h>

#include <string>

#include "irm_attn.h"
#include "irm_launch.h"

namespace irm {
namespace {

using namespace irm::dev;

// ---------------------------------------------------------------------------
// Four queries per workgroup, one 16-head group: the four (query, 16 heads)
// groups share every 32-row tile of the causal range of the last query.
// Scoring wave s scores query s; accumulating wave j copies and rotates
// slice j of every tile and sums output columns 128 j .. 128 j + 127 of all
// four queries (score_stream / value_stream).
// ---------------------------------------------------------------------------
constexpr uint32_t kQueriesPerBlock = kSplitGroups;

struct PrefillArgs {
  StreamArgs ra;
  const uint32_t* seq_base;
  const uint4* q_lat;
  const uint4* q_rope;
  uint16_t* out;
  float* lse;
  uint32_t n_q, n_heads, n_groups;
  int32_t q_pos0;
  float scale_log2;
  InvFreq f;
};

// kFlat: the KV is an assembled cache (row = position, every delta 0), read
// without row map or rotation; otherwise rows come through the chunk table.
template <bool kFlat>
__global__ __launch_bounds__(kRoleThreads, 1) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) SplitSmem sm;

  const uint32_t hg = blockIdx.x % a.n_groups;
  const uint32_t q0 = (blockIdx.x / a.n_groups) * kQueriesPerBlock;
  const uint32_t lane = threadIdx.x & 63, w = wave_id(), hq = lane >> 4, hr = lane & 15;
  const uint32_t head = hg * 16 + hr;
  const uint32_t q_last = min(a.n_q, q0 + kQueriesPerBlock) - 1;
  const uint32_t rows = (uint32_t)a.q_pos0 + q_last + 1;  // KV rows this workgroup visits
  fill_omega(sm.s.omega, a.f);

  if (w < kSplitGroups) {  // scoring wave: query q0 + w
    const uint32_t qi = q0 + w;
    const int64_t lim = qi < a.n_q ? (int64_t)a.q_pos0 + qi : -1;  // last visible row of the query
    bf16x8_t qb[18];
    load_q<false>(a.q_lat, a.q_rope, min(qi, q_last), a.n_heads, head, qb);
    float m = -INFINITY, l = 0.f;
    __syncthreads();
    score_stream<kFlat>(a.ra, sm, kFlat ? 0u : a.seq_base[0], rows, a.scale_log2,
                 [&](uint32_t t, uint32_t) -> int32_t {
                   const int64_t last = lim - (int64_t)t * kTileRows;
                   return last > kTileRows ? kTileRows : (last < -1 ? -1 : (int32_t)last);
                 },
                 qb, m, l);
    split_publish(sm, m, l);
    if (a.lse && qi < a.n_q && hq == 0)
      a.lse[(size_t)qi * a.n_heads + head] = (sm.ml[w][hr][0] + log2f(sm.ml[w][hr][1])) * kLn2;
    return;
  }

  // accumulating wave j: columns 128 j .. 128 j + 127 of the four queries
  const uint32_t j = w - kSplitGroups;
  f32x4_t o[kSplitGroups][kSplitNb];
#pragma unroll
  for (int g = 0; g < kSplitGroups; ++g)
#pragma unroll
    for (int nb = 0; nb < kSplitNb; ++nb) o[g][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  value_stream<kFlat>(a.ra, sm, kFlat ? 0u : a.seq_base[0], rows, o);
  split_publish_wait();
#pragma unroll
  for (int g = 0; g < kSplitGroups; ++g) {
    const uint32_t qg = q0 + g;
    if (qg >= a.n_q) break;
    const float inv = 1.f / sm.ml[g][hr][1];
    uint16_t* op = a.out + ((size_t)qg * a.n_heads + head) * IRM_D_LATENT + kSplitCols * j + 4 * hq;
#pragma unroll
    for (int nb = 0; nb < kSplitNb; ++nb) {
      uint2 v;
      v.x = pack_bf16(o[g][nb][0] * inv, o[g][nb][1] * inv);
      v.y = pack_bf16(o[g][nb][2] * inv, o[g][nb][3] * inv);
      *reinterpret_cast<uint2*>(op + 16 * nb) = v;
    }
  }
}

}  // namespace

namespace {

PrefillArgs prefill_args(const void* q_lat, const void* q_rope, int32_t q_pos0, uint32_t n_q, const void* pool,
                         uint64_t pool_rows, uint32_t n_heads, float scale, void* out, float* lse) {
  PrefillArgs a{};
  a.ra.pool = static_cast<const unsigned char*>(pool);
  a.ra.pool_last = pool_last_of(pool_rows);
  a.q_lat = static_cast<const uint4*>(q_lat);
  a.q_rope = static_cast<const uint4*>(q_rope);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.n_q = n_q;
  a.n_heads = n_heads;
  a.n_groups = n_heads / 16;
  a.q_pos0 = q_pos0;
  a.scale_log2 = scale * kLog2e;
  return a;
}

template <bool kFlat>
irm_status launch(const PrefillArgs& a, hipStream_t s, const char* fn) {
  const uint64_t grid = (uint64_t)(a.n_q + kQueriesPerBlock - 1) / kQueriesPerBlock * a.n_groups;
  if (grid > 0x7fffffffull) return fail(IRM_EUNSUPPORTED, std::string(fn) + ": grid too large");
  hipLaunchKernelGGL(prefill_kernel<kFlat>, dim3((uint32_t)grid), dim3(kRoleThreads), 0, s, a);
  return launch_check(fn);
}

}  // namespace

irm_status launch_prefill(const irm_table* t, const void* q_lat, const void* q_rope, int32_t q_pos0,
                          uint32_t n_q, const void* pool, uint64_t pool_rows, uint32_t n_heads, float scale,
                          void* out, float* lse, hipStream_t s) {
  PrefillArgs a = prefill_args(q_lat, q_rope, q_pos0, n_q, pool, pool_rows, n_heads, scale, out, lse);
  a.ra.rowmap = image_of(t).rowmap;
  a.ra.trig = image_of(t).trig;
  a.seq_base = image_of(t).seq_base;
  for (int i = 0; i < (int)kPairs; ++i) a.f.w[i] = t->inv_freq[i];
  return launch<false>(a, s, "irm_mla_prefill_tail");
}

irm_status launch_prefill_assembled(const void* q_lat, const void* q_rope, int32_t q_pos0, uint32_t n_q,
                                    const void* kv, uint64_t kv_rows, uint32_t n_heads, float scale, void* out,
                                    float* lse, hipStream_t s) {
  const PrefillArgs a = prefill_args(q_lat, q_rope, q_pos0, n_q, kv, kv_rows, n_heads, scale, out, lse);
  return launch<true>(a, s, "irm_mla_prefill_assembled");
}

}  // namespace irm
