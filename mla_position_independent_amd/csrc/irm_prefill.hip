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
// register tile pipeline (tail-prefill)
//
// Four waves share every 64-row tile: rows are loaded into registers one
// tile ahead (rotated there with the per-entry trig table), stored to a
// padded LDS tile, and scored by all four waves against their own queries.
// LDS rows are padded to kLdsRow bytes.
// ---------------------------------------------------------------------------
constexpr int kLdsRow = kRowBytes + 32;  // padded LDS row stride

// One 64-row KV tile in registers.  Thread (wave w, lane l) holds c_KV unit l
// of rows 16w + k (k = 0..15) and k_r unit tid % 8 of rows tid / 8 and
// 32 + tid / 8 (every c_KV load instruction of a wave reads 1 KB of one row),
// plus the (cos, sin) of the 4 pairs of each k_r unit.
struct TileRegs {
  u32x4_t c[16];
  u32x4_t kr[2];
  f32x4_t tr[2][2];
  uint32_t rot;  // bit j: k_r unit j is rotated
};

// Row-map record of tile row tid (threads 0..63): {pool row, entry or kNoRot}.
// Rows past the end map to pool row 0 (any valid row: their scores are
// masked, and finite data keeps 0 * value = 0 in the PV product).
__device__ __forceinline__ uint2 load_rowmap(const uint4* __restrict__ rowmap, uint32_t g0,
                                             uint32_t nrows) {
  const uint32_t t = threadIdx.x;
  if (t >= nrows) return make_uint2(0u, kNoRot);
  const uint4 r = rowmap[g0 + t];
  return make_uint2(r.x, r.z);
}

__device__ __forceinline__ void put_rowmap(uint2 rec, uint32_t* s_src, uint32_t* s_rot) {
  if (threadIdx.x < kTile) {
    s_src[threadIdx.x] = rec.x;
    s_rot[threadIdx.x] = rec.y;
  }
}

// Issue the global loads of one tile, branch free so that all of them are in
// flight together.  Pool rows and entries come from the validated row map;
// they are also clamped so that a corrupted map shows up as a wrong result,
// never as a fault.
__device__ __forceinline__ void issue_tile(const uint4* __restrict__ pool, uint32_t pool_last,
                                           const float2* __restrict__ trig, uint32_t ent_last,
                                           const uint32_t* s_src, const uint32_t* s_rot, TileRegs& v) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const u32x4_t* P = reinterpret_cast<const u32x4_t*>(pool);
  const u32x4_t* rows = reinterpret_cast<const u32x4_t*>(s_src + 16 * w);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4_t x = rows[q];
#pragma unroll
    for (int i = 0; i < 4; ++i) v.c[4 * q + i] = P[(size_t)min(x[i], pool_last) * kUnitsPerRow + l];
  }
  v.rot = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t r = (threadIdx.x >> 3) + 32 * j;
    const uint32_t e = s_rot[r];
    v.kr[j] = P[(size_t)min(s_src[r], pool_last) * kUnitsPerRow + kLatUnits + (threadIdx.x & 7)];
    const f32x4_t* tp = reinterpret_cast<const f32x4_t*>(trig + (size_t)min(e, ent_last) * irm::kPairs +
                                                         (threadIdx.x & 7) * 4);
    v.tr[j][0] = tp[0];
    v.tr[j][1] = tp[1];
    v.rot |= (e != kNoRot ? 1u : 0u) << j;
  }
}

__device__ __forceinline__ void rotate_tile(TileRegs& v) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const f32x4_t a = v.tr[j][0], b = v.tr[j][1];
    const u32x4_t k = v.kr[j];
    const u32x4_t r = {rotate_pair(k[0], a[0], a[1]), rotate_pair(k[1], a[2], a[3]),
                       rotate_pair(k[2], b[0], b[1]), rotate_pair(k[3], b[2], b[3])};
    v.kr[j] = ((v.rot >> j) & 1u) ? r : k;
  }
}

__device__ __forceinline__ void store_tile_lds(unsigned char* lds, const TileRegs& v) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < 16; ++k) *reinterpret_cast<u32x4_t*>(lds + (16 * w + k) * kLdsRow + 16 * l) = v.c[k];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    *reinterpret_cast<u32x4_t*>(lds + ((threadIdx.x >> 3) + 32 * j) * kLdsRow + 2 * IRM_D_LATENT +
                                16 * (threadIdx.x & 7)) = v.kr[j];
}

// Shared memory of the tile pipeline.
struct TileSmem {
  unsigned char tile[kTile * kLdsRow];
  uint32_t src[3][kTile];
  uint32_t rot[3][kTile];
};

// Stream the assembled rows [g_begin, g_begin + n) through LDS in 64-row
// tiles, calling compute(t, nrows) with tile t resident in sm.tile.  With
// kDepth = 2 the loads of tiles t+1 and t+2 are in flight while tile t is
// computed (two register sets); with kDepth = 1 only tile t+1 is.  The row
// map runs kDepth + 1 tiles ahead in LDS and one more in registers.  Every
// thread of the workgroup must call this with the same arguments.
template <int kDepth, class Compute>
__device__ __forceinline__ void stream_tiles(const Image& im, const uint4* __restrict__ rowmap,
                                             const uint4* __restrict__ pool, uint32_t pool_last,
                                             uint32_t g_begin, uint32_t n, TileSmem& sm, Compute&& compute) {
  static_assert(kDepth == 1 || kDepth == 2, "pipeline depth 1 or 2");
  const uint32_t ntiles = (n + kTile - 1) / kTile;
  if (ntiles == 0) return;
  auto rows_of = [&](uint32_t t) { return min((uint32_t)kTile, n - t * kTile); };
  for (uint32_t t = 0; t <= (uint32_t)kDepth && t < ntiles; ++t)
    put_rowmap(load_rowmap(rowmap, g_begin + t * kTile, rows_of(t)), sm.src[t % 3], sm.rot[t % 3]);
  __syncthreads();
  TileRegs va, vb;
  issue_tile(pool, pool_last, im.trig, im.n_entries - 1, sm.src[0], sm.rot[0], va);
  if (kDepth == 2 && ntiles > 1) issue_tile(pool, pool_last, im.trig, im.n_entries - 1, sm.src[1], sm.rot[1], vb);
  uint2 ri = make_uint2(0u, kNoRot);
  if (ntiles > kDepth + 1) ri = load_rowmap(rowmap, g_begin + (kDepth + 1) * kTile, rows_of(kDepth + 1));

  // one pipeline step on register set v (which holds tile t)
#define IRM_PIPE_STEP(t, v)                                                                          \
  do {                                                                                               \
    rotate_tile(v);                                                                                  \
    __syncthreads(); /* every wave is done with tile t-1 */                                          \
    store_tile_lds(sm.tile, v);                                                                      \
    /* the row map of tile x always lives in slot x % 3 */                                           \
    if ((t) + kDepth + 1 < ntiles)                                                                   \
      put_rowmap(ri, sm.src[((t) + kDepth + 1) % 3], sm.rot[((t) + kDepth + 1) % 3]);                \
    __syncthreads(); /* tile t and the row map of tile t+kDepth+1 are visible */                     \
    const uint32_t tn = (t) + kDepth;                                                                \
    if (tn < ntiles) issue_tile(pool, pool_last, im.trig, im.n_entries - 1, sm.src[tn % 3], sm.rot[tn % 3], v); \
    if (tn + 2 < ntiles) ri = load_rowmap(rowmap, g_begin + (tn + 2) * kTile, rows_of(tn + 2));     \
    compute((t), rows_of(t));                                                                        \
  } while (0)
  if constexpr (kDepth == 1) {
    for (uint32_t t = 0; t < ntiles; ++t) IRM_PIPE_STEP(t, va);
  } else {
    for (uint32_t t = 0; t < ntiles; t += 2) {
      IRM_PIPE_STEP(t, va);
      if (t + 1 < ntiles) IRM_PIPE_STEP(t + 1, vb);
    }
  }
#undef IRM_PIPE_STEP
}

// S^T for the four 16-row blocks of a tile: lane (q = lane/16, r = lane%16)
// gets in acc[j] the scores of rows 16j + 4q + i (i = 0..3) for head r.  The
// four blocks are interleaved so that LDS reads overlap independent MFMAs.
__device__ __forceinline__ void qk_tile(const unsigned char* lds, const bf16x8_t (&qb)[18],
                                        f32x4_t (&acc)[4]) {
  const int lane = threadIdx.x & 63;
  const unsigned char* p = lds + (lane & 15) * kLdsRow + (lane >> 4) * 16;
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    bf16x8_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p + 16 * j * kLdsRow + kk * 64));
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], qb[kk], acc[j], 0, 0, 0);
  }
}

// PV over a pair of 16-row blocks on v_mfma_f32_16x16x32_bf16:
// O^T[n][head] += C^T[n][k] P^T[k][head], k = 32 tile rows.  The A operand
// (8 consecutive k per lane) comes from two transposing LDS reads
// (ds_read_b64_tr_b16): within each 16-lane group, lane 4a+b receives element
// b of the 8-byte reads of lanes a, a+4, a+8, a+12.  Lane (q, s) therefore
// reads row row0 + 4q + s/4, columns n0 + 4(s%4)..+3, and gets C[row0 + 4q + i]
// [n0 + s] for i = 0..3; the second read covers rows row0 + 16 + 4q + i.  The
// k order {4q..4q+3, 16+4q..16+4q+3} matches the lane's P^T values of the two
// score blocks, so pb is just those 8 probabilities.
typedef short i16x4_lds_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8_t tr_pair(const unsigned char* p0, const unsigned char* p1) {
  typedef __attribute__((address_space(3))) i16x4_lds_t* lds_ptr_t;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr_t)(p0));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr_t)(p1));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int NB>
__device__ __forceinline__ void pv_pair(const unsigned char* lds, int row0, int nb0, bf16x8_t pb,
                                        f32x4_t (&o)[NB]) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, s = lane & 15;
  const unsigned char* p0 = lds + (row0 + 4 * q + (s >> 2)) * kLdsRow + 8 * (s & 3) + 32 * nb0;
  const unsigned char* p1 = p0 + 16 * kLdsRow;
  // reads in groups of eight column blocks, each group issued ahead of its MFMAs
  constexpr int kGroup = NB < 8 ? NB : 8;
#pragma unroll
  for (int g0 = 0; g0 < NB; g0 += kGroup) {
    bf16x8_t a[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) a[j] = tr_pair(p0 + 32 * (g0 + j), p1 + 32 * (g0 + j));
#pragma unroll
    for (int j = 0; j < kGroup; ++j) o[g0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], pb, o[g0 + j], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// chunked tail-prefill: 4 queries per workgroup (one per wave), 16 heads
// ---------------------------------------------------------------------------
struct PrefillArgs {
  Image im;
  const uint4* pool;
  const uint4* q_lat;
  const uint4* q_rope;
  uint16_t* out;
  float* lse;
  uint32_t n_q, n_heads, n_groups;
  uint32_t pool_last;  // last valid pool row
  int32_t q_pos0;
  float scale_log2;
};

__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) TileSmem sm;

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
  f32x4_t o[32];
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  stream_tiles<1>(a.im, a.im.rowmap, a.pool, a.pool_last, a.im.seq_base[0], rows, sm, [&](uint32_t t, uint32_t) {
    const int64_t t0 = (int64_t)t * kTile;
    if (t0 > lim) return;
    f32x4_t acc[4];
    qk_tile(sm.tile, qb, acc);
    float sc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[j][i] = (t0 + 16 * j + 4 * hq + i <= lim) ? acc[j][i] * a.scale_log2 : -INFINITY;
    float p[4][4];
    softmax_update_n<4, 32>(sc, m, l, o, p);
    pv_pair<32>(sm.tile, 0, 0, pack_p8(p[0], p[1]), o);
    if (t0 + 32 <= lim) pv_pair<32>(sm.tile, 32, 0, pack_p8(p[2], p[3]), o);
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
  a.im = image_of(t);
  a.pool = static_cast<const uint4*>(pool);
  a.q_lat = static_cast<const uint4*>(q_lat);
  a.q_rope = static_cast<const uint4*>(q_rope);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.n_q = n_q;
  a.n_heads = n_heads;
  a.pool_last = pool_last_of(pool_rows);
  a.n_groups = n_heads / 16;
  a.q_pos0 = q_pos0;
  a.scale_log2 = scale * kLog2e;
  const uint64_t grid = (uint64_t)(n_q + 3) / 4 * a.n_groups;
  if (grid > 0x7fffffffull) return fail(IRM_EUNSUPPORTED, "irm_mla_prefill_tail: grid too large");
  hipLaunchKernelGGL(prefill_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, s, a);
  return launch_check("irm_mla_prefill_tail");
}

}  // namespace irm
