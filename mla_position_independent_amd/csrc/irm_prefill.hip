// Chunked tail-prefill: causal absorbed MLA attention of a block of new
// query tokens over the assembled cache, with the delta rotation applied as
// KV rows are loaded (Irminsul pages: gentlecold.top article, sections 4, 5
// and 15; gist.science summary, section 2.2).

#include <hip/hip_runtime.h>

#include "irm_attn.h"
#include "irm_launch.h"

namespace irm {
namespace {

using namespace irm::dev;

// ---------------------------------------------------------------------------
// Four queries per workgroup (one per wave), 16 heads.  The four waves share
// every 32-row tile of the causal range of their last query (shared_stream:
// each wave copies and rotates one 8-row slice); a wave skips the tiles
// that lie wholly past its own query and masks the rest on absolute
// position.
// ---------------------------------------------------------------------------
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

__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) SharedSmem sm;

  const uint32_t g = blockIdx.x % a.n_groups;
  const uint32_t qblk = blockIdx.x / a.n_groups;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hq = lane >> 4, hr = lane & 15;
  const uint32_t head = g * 16 + hr;
  const uint32_t qi = qblk * 4 + wave;
  const bool active = qi < a.n_q;
  const uint32_t q_last = min(a.n_q, qblk * 4 + 4) - 1;
  const uint32_t rows = (uint32_t)a.q_pos0 + q_last + 1;   // KV rows this workgroup visits
  const int64_t lim = active ? (int64_t)a.q_pos0 + qi : -1;  // last visible row of this wave

  bf16x8_t qb[18];
  load_q(a.q_lat, a.q_rope, active ? qi : q_last, a.n_heads, head, qb);
  fill_omega(sm.omega, a.f);
  f32x4_t o[32];
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  __syncthreads();

  shared_stream(a.ra, sm, a.seq_base[0], rows, [&](const unsigned char* st, uint32_t t, uint32_t) {
    const int64_t t0 = (int64_t)t * kTileRows;
    if (t0 > lim) return;
    f32x4_t acc[2];
    qk_blocks<2>(st, st + kTileKr, 0, qb, acc);
    float sc[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[j][i] = acc[j][i];
    if (t0 + kTileRows - 1 > lim) {  // the causal edge runs through this tile
      const int32_t last = (int32_t)(lim - t0);  // last visible tile row
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * j + 4 * hq + i > last) sc[j][i] = -INFINITY;
    }
    float p[2][4];
    softmax_update_n<2, 32>(sc, a.scale_log2, m, l, o, p);
    pv_pair<32>(st, 0, 0, pack_p8(p[0], p[1]), o);
  });

  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (!active) return;
  const float inv = 1.f / l;
  uint16_t* op = a.out + ((size_t)qi * a.n_heads + head) * IRM_D_LATENT + 4 * hq;
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) {
    uint2 w;
    w.x = pack_bf16(o[nb][0] * inv, o[nb][1] * inv);
    w.y = pack_bf16(o[nb][2] * inv, o[nb][3] * inv);
    *reinterpret_cast<uint2*>(op + 16 * nb) = w;
  }
  if (a.lse && hq == 0) a.lse[(size_t)qi * a.n_heads + head] = (m + log2f(l)) * kLn2;
}

}  // namespace

irm_status launch_prefill(const irm_table* t, const void* q_lat, const void* q_rope, int32_t q_pos0,
                          uint32_t n_q, const void* pool, uint64_t pool_rows, uint32_t n_heads, float scale,
                          void* out, float* lse, hipStream_t s) {
  PrefillArgs a;
  a.ra.pool = static_cast<const unsigned char*>(pool);
  a.ra.rowmap = image_of(t).rowmap;
  a.ra.pool_last = pool_last_of(pool_rows);
  a.seq_base = image_of(t).seq_base;
  a.q_lat = static_cast<const uint4*>(q_lat);
  a.q_rope = static_cast<const uint4*>(q_rope);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.n_q = n_q;
  a.n_heads = n_heads;
  a.n_groups = n_heads / 16;
  a.q_pos0 = q_pos0;
  a.scale_log2 = scale * kLog2e;
  for (int i = 0; i < (int)kPairs; ++i) a.f.w[i] = t->inv_freq[i];
  const uint64_t grid = (uint64_t)(n_q + 3) / 4 * a.n_groups;
  if (grid > 0x7fffffffull) return fail(IRM_EUNSUPPORTED, "irm_mla_prefill_tail: grid too large");
  hipLaunchKernelGGL(prefill_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, s, a);
  return launch_check("irm_mla_prefill_tail");
}

}  // namespace irm
