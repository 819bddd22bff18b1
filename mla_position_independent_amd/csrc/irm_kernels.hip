// HIP kernels (gfx950) and the C ABI entry points that launch them.
//
// Operations follow the Irminsul pages (arXiv:2605.05696):
//  * delta rotation k_r = R(p_tgt - p_src) k_r_base of the 64-wide RoPE slice,
//    with c_KV reused unchanged (gist.science summary 2.1-2.2; gentlecold.top
//    article sections 4, 5 and 15);
//  * absorbed MLA attention: score = q_lat . c_KV + q_rope . k_r, value = c_KV
//    (gentlecold.top section 4), rotating k_r while the KV tile is loaded, the
//    fusion the pages propose for the HBM-to-on-chip load (gist.science 2.2
//    and 4; gentlecold.top sections 5 and 14.1).
//
// Data layout: pool and assembled rows are bf16 [rows][576] = 72 units of
// 16 bytes; units 0..63 are c_KV, units 64..71 are k_r (4 rotation pairs per
// unit).  Angles are formed and their sine/cosine evaluated in double once per
// table entry (delta reaches 2^17, where a float angle is off by ~1e-2 rad);
// only the 2x2 rotation itself runs in float.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <string>

#include "irm_internal.h"

using irm::DevEntry;
using irm::fail;

namespace {

constexpr int kRowBytes = IRM_ROW * 2;                       // 1152
constexpr int kUnitsPerRow = kRowBytes / 16;                 // 72
constexpr int kLatUnits = IRM_D_LATENT * 2 / 16;             // 64
constexpr int kThreads = 256;                                // 4 waves of 64
constexpr int kTile = 64;                                    // KV rows per tile
constexpr int kUnitsPerThread = kTile * kUnitsPerRow / kThreads;  // 18
constexpr int kLdsRow = kRowBytes + 32;                      // padded LDS row stride
constexpr uint32_t kNoRot = 0xffffffffu;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct InvFreq {
  double w[irm::kPairs];
};

struct Image {
  const DevEntry* ents;
  const uint32_t* seq_first;
  const uint32_t* seq_base;
  const uint32_t* block_map;
  const float2* trig;
  const uint2* rowmap;
  uint32_t n_entries;
};

Image image_of(const irm_table* t) {
  const unsigned char* d = static_cast<const unsigned char*>(t->dev);
  Image im;
  im.ents = reinterpret_cast<const DevEntry*>(d + t->layout.off_entries);
  im.seq_first = reinterpret_cast<const uint32_t*>(d + t->layout.off_seq_first);
  im.seq_base = reinterpret_cast<const uint32_t*>(d + t->layout.off_seq_base);
  im.block_map = reinterpret_cast<const uint32_t*>(d + t->layout.off_block_map);
  im.trig = reinterpret_cast<const float2*>(d + t->layout.off_trig);
  im.rowmap = reinterpret_cast<const uint2*>(d + t->layout.off_rowmap);
  im.n_entries = t->n_chunks;
  return im;
}

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (inputs are finite)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// Entry that holds assembled row g: start at the block map, walk forward.
__device__ __forceinline__ uint32_t find_entry(const Image& im, uint32_t g) {
  uint32_t e = im.block_map[g / irm::kBlockRows];
  while (g >= im.ents[e].out_row + im.ents[e].len) ++e;
  return e;
}

// Rotate the 4 pairs of one k_r unit; pair p uses (cos, sin) = tr[p].
// x' = x cos - y sin, y' = x sin + y cos, in float.
__device__ __forceinline__ void rotate_unit_f32(const uint4& w, const float2* tr, float (&f)[8]) {
  const uint32_t word[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float x = bf16_lo(word[p]), y = bf16_hi(word[p]);
    const float2 cs = tr[p];
    f[2 * p] = fmaf(x, cs.x, -(y * cs.y));
    f[2 * p + 1] = fmaf(x, cs.y, y * cs.x);
  }
}

__device__ __forceinline__ uint4 rotate_unit(const uint4& w, const float2* tr) {
  float f[8];
  rotate_unit_f32(w, tr, f);
  return make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]),
                    pack_bf16(f[6], f[7]));
}

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
// row map: {pool row, entry if rotated else kNoRot} per assembled row
// ---------------------------------------------------------------------------
__global__ void rowmap_kernel(Image im, uint32_t total_rows, uint2* __restrict__ rowmap) {
  const uint32_t g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= total_rows) return;
  const uint32_t e = find_entry(im, g);
  const DevEntry d = im.ents[e];
  rowmap[g] = make_uint2(d.pool_row + (g - d.out_row), d.delta != 0 ? e : kNoRot);
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

// ---------------------------------------------------------------------------
// attention building blocks (shared by decode and tail-prefill)
//
// A workgroup of 4 waves streams KV tiles of 64 rows through LDS (padded
// row-major, c_KV and rotated k_r).  Tile t+1 is loaded into registers while
// tile t is computed; the row map of tile t+2 is already in LDS and that of
// tile t+3 is in flight, so no dependent table lookup sits on the critical
// path.  k_r is rotated in registers between the global load and the LDS
// store, with the entry's (cos, sin) fetched together with the data.
//
// The score block of 16 rows x 16 heads is S^T = K Q^T on
// v_mfma_f32_16x16x32_bf16 (K from LDS, Q^T from registers), so each lane
// ends with 4 rows of one head; O^T = C^T P^T then leaves every lane with
// outputs of a single head, so the online-softmax rescale is lane-local.
// Softmax runs in the base-2 domain (scores pre-multiplied by scale*log2 e).
// ---------------------------------------------------------------------------

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
__device__ __forceinline__ uint2 load_rowmap(const uint2* __restrict__ rowmap, uint32_t g0,
                                             uint32_t nrows) {
  const uint32_t t = threadIdx.x;
  return (t < nrows) ? rowmap[g0 + t] : make_uint2(0u, kNoRot);
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

// One rotation pair: (x, y) packed as bf16 in w, (cos, sin) = (c, s).
__device__ __forceinline__ uint32_t rotate_pair(uint32_t w, float c, float s) {
  const float x = bf16_lo(w), y = bf16_hi(w);
  return pack_bf16(fmaf(x, c, -(y * s)), fmaf(x, s, y * c));
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
__device__ __forceinline__ void stream_tiles(const Image& im, const uint2* __restrict__ rowmap,
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

// Q^T operands of one head group for one query: lane (q, r) holds head
// g*16 + r, dims 32 kk + 8 q .. +8 (kk 0..15 latent, 16..17 rope).
__device__ __forceinline__ void load_q(const uint4* __restrict__ q_lat, const uint4* __restrict__ q_rope,
                                       uint32_t qrow, uint32_t n_heads, uint32_t head,
                                       bf16x8_t (&qb)[18]) {
  const int q = (threadIdx.x & 63) >> 4;
  const uint4* pl = q_lat + ((size_t)qrow * n_heads + head) * (IRM_D_LATENT / 8) + q;
  const uint4* pr = q_rope + ((size_t)qrow * n_heads + head) * (IRM_D_ROPE / 8) + q;
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) qb[kk] = __builtin_bit_cast(bf16x8_t, pl[4 * kk]);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) qb[16 + kk] = __builtin_bit_cast(bf16x8_t, pr[4 * kk]);
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
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const bf16x8_t a = tr_pair(p0 + 32 * nb, p1 + 32 * nb);
    o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[nb], 0, 0, 0);
  }
}

template <int NB, int NO>
__device__ __forceinline__ void softmax_update_n(float (&s)[NB][4], float& m, float& l,
                                                 f32x4_t (&o)[NO], float (&p)[NB][4]) {
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[j][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(m, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = exp2f(m - m_use);  // m == -inf gives 0
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[j][i] = exp2f(s[j][i] - m_use);
      sum += p[j][i];
    }
  l = l * alpha + sum;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int nb = 0; nb < NO; ++nb) o[nb] *= alpha;
  }
  m = m_new;
}

__device__ __forceinline__ bf16x8_t pack_p8(const float (&a)[4], const float (&b)[4]) {
  const uint4 w = make_uint4(pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]),
                             pack_bf16(b[2], b[3]));
  return __builtin_bit_cast(bf16x8_t, w);
}

// ---------------------------------------------------------------------------
// split-KV decode, pass 1
//
// Workgroup = (sequence, split, block of HG head groups of 16), 4 waves.
// Wave w serves head group w / CG and output columns [512/CG * (w % CG), ..):
// every wave scores all 64 rows of a tile for its 16 heads (the CG waves of a
// head group repeat the same score work and reach bit-identical softmax
// state), then accumulates only its column slice, so each lane holds 128/CG
// accumulators and no cross-wave merge is needed.
// ---------------------------------------------------------------------------
// Tile pipeline depth of the decode kernel: 1 = one tile in flight with two
// workgroups per CU, 2 = two tiles in flight with one workgroup per CU.
constexpr int kDecodeDepth = 1;

struct DecodeArgs {
  Image im;
  const uint4* pool;
  const uint4* q_lat;
  const uint4* q_rope;
  float* ws_acc;  // [n_seq][n_splits][n_heads][512], unnormalised
  float* ws_ml;   // [n_seq][n_splits][n_heads][2]: base-2 max, sum
  uint32_t n_seq, n_heads, n_gblocks, n_splits;
  uint32_t pool_last;  // last valid pool row
  float scale_log2;
};

template <int HG, int CG, int kDepth>
__global__ __launch_bounds__(kThreads, 3 - kDepth) void decode_split_kernel(DecodeArgs a) {
  static_assert(HG * CG == kThreads / 64, "one wave per (head group, column group)");
  constexpr int kNB = 32 / CG;  // 16-column output blocks per wave
  __shared__ __attribute__((aligned(16))) TileSmem sm;

  // Workgroups of the same (sequence, split) but different head-group blocks
  // get the same x % 8, i.e. the same XCD and L2, at consecutive slots.
  const uint32_t x = blockIdx.x, xcd = x & 7, slot = x >> 3;
  const uint32_t gb = slot % a.n_gblocks;
  const uint32_t bs = (slot / a.n_gblocks) * 8 + xcd;
  if (bs >= a.n_seq * a.n_splits) return;
  const uint32_t b = bs / a.n_splits, sp = bs % a.n_splits;

  const uint32_t base = a.im.seq_base[b];
  const uint32_t N = a.im.seq_base[b + 1] - base;
  const uint32_t per = ((N + a.n_splits - 1) / a.n_splits + kTile - 1) / kTile * kTile;
  const uint32_t r0 = min(N, sp * per), r1 = min(N, r0 + per);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hq = lane >> 4, hr = lane & 15;
  const int hg = wave / CG, cg = wave % CG;
  const uint32_t head = (gb * HG + hg) * 16 + hr;

  bf16x8_t qb[18];
  load_q(a.q_lat, a.q_rope, b, a.n_heads, head, qb);

  f32x4_t o[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  stream_tiles<kDepth>(a.im, a.im.rowmap, a.pool, a.pool_last, base + r0, r1 - r0, sm, [&](uint32_t, uint32_t nrows) {
    f32x4_t acc[4];
    qk_tile(sm.tile, qb, acc);
    float sc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc[j][i] = ((uint32_t)(16 * j + 4 * hq + i) < nrows) ? acc[j][i] * a.scale_log2 : -INFINITY;
    float p[4][4];
    softmax_update_n<4, kNB>(sc, m, l, o, p);
    pv_pair<kNB>(sm.tile, 0, cg * kNB, pack_p8(p[0], p[1]), o);
    if (nrows > 32) pv_pair<kNB>(sm.tile, 32, cg * kNB, pack_p8(p[2], p[3]), o);
  });

  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const size_t pidx = ((size_t)b * a.n_splits + sp) * a.n_heads + head;
  float* dst = a.ws_acc + pidx * IRM_D_LATENT + 16 * cg * kNB + 4 * hq;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
    *reinterpret_cast<float4*>(dst + 16 * nb) = make_float4(o[nb][0], o[nb][1], o[nb][2], o[nb][3]);
  if (cg == 0 && hq == 0) {
    a.ws_ml[pidx * 2 + 0] = m;
    a.ws_ml[pidx * 2 + 1] = (m == -INFINITY) ? 0.f : l;
  }
}

// ---------------------------------------------------------------------------
// split-KV decode, pass 2: merge the splits of each (sequence, head)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ ws_acc,
                                                             const float* __restrict__ ws_ml,
                                                             uint16_t* __restrict__ out,
                                                             float* __restrict__ lse,
                                                             uint32_t n_heads, uint32_t n_splits) {
  const uint32_t bh = blockIdx.x;
  const uint32_t b = bh / n_heads, h = bh % n_heads;
  float mx = -INFINITY;
  for (uint32_t s = 0; s < n_splits; ++s)
    mx = fmaxf(mx, ws_ml[(((size_t)b * n_splits + s) * n_heads + h) * 2]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (uint32_t s = 0; s < n_splits; ++s) {
    const size_t p = ((size_t)b * n_splits + s) * n_heads + h;
    const float ms = ws_ml[p * 2];
    if (ms == -INFINITY) continue;
    const float f = exp2f(ms - mx);
    L += f * ws_ml[p * 2 + 1];
    const float4 v = reinterpret_cast<const float4*>(ws_acc + p * IRM_D_LATENT)[threadIdx.x];
    acc.x += f * v.x;
    acc.y += f * v.y;
    acc.z += f * v.z;
    acc.w += f * v.w;
  }
  const float inv = 1.f / L;
  uint2 w;
  w.x = pack_bf16(acc.x * inv, acc.y * inv);
  w.y = pack_bf16(acc.z * inv, acc.w * inv);
  reinterpret_cast<uint2*>(out + (size_t)bh * IRM_D_LATENT)[threadIdx.x] = w;
  if (lse && threadIdx.x == 0) lse[bh] = (mx + log2f(L)) * kLn2;
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

// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------
irm_status hip_check(hipError_t err, const char* what) {
  if (err == hipSuccess) return IRM_OK;
  return fail(IRM_EHIP, std::string(what) + ": " + hipGetErrorString(err));
}

irm_status launch_check(const char* what) { return hip_check(hipGetLastError(), what); }

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

// Head groups of 16 handled by one decode workgroup for G = n_heads / 16.
uint32_t heads_per_block(uint32_t G) { return (G % 2 == 0 && G < 4) ? 2 : 1; }

uint32_t default_splits(const irm_table* t, uint32_t n_groups) {
  // aim for >= 2 workgroups per CU (256 CUs) with >= 256 rows per split
  const uint32_t want = (512 + t->n_seq * n_groups - 1) / (t->n_seq * n_groups);
  const uint32_t cap = (t->max_seq_len + 255) / 256;
  uint32_t s = want < cap ? want : cap;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return s;
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
  if (t->total_rows) {
    const uint32_t n = (uint32_t)t->total_rows;
    const Image im = image_of(t);
    hipLaunchKernelGGL(rowmap_kernel, dim3((n + 255) / 256), dim3(256), 0, s, im, n,
                       const_cast<uint2*>(im.rowmap));
    st = launch_check("irm_table_upload: row map kernel");
    if (st != IRM_OK) { t->dev = nullptr; return st; }
  }
  st = irm_table_set_rope(t, inv_freq, stream);
  if (st != IRM_OK) t->dev = nullptr;
  return st;
}

extern "C" irm_status irm_table_set_rope(irm_table* t, const double* inv_freq, void* stream) {
  irm_status st = need_uploaded(t, "irm_table_set_rope");
  if (st != IRM_OK) return st;
  if (!inv_freq) return fail(IRM_EINVAL, "irm_table_set_rope: inv_freq is NULL");
  for (int i = 0; i < (int)irm::kPairs; ++i)
    if (!std::isfinite(inv_freq[i])) return fail(IRM_EINVAL, "irm_table_set_rope: inv_freq not finite");
  if (!t->n_chunks) return IRM_OK;
  InvFreq f;
  std::memcpy(f.w, inv_freq, sizeof(f.w));
  const uint32_t n = t->n_chunks * irm::kPairs;
  const Image im = image_of(t);
  hipLaunchKernelGGL(trig_kernel, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                     im.ents, t->n_chunks, f, const_cast<float2*>(im.trig));
  return launch_check("irm_table_set_rope: trig kernel");
}

extern "C" irm_status irm_table_gather_index(const irm_table* t, int64_t* pool_row, int32_t* delta,
                                             void* stream) {
  irm_status st = need_uploaded(t, "irm_table_gather_index");
  if (st != IRM_OK) return st;
  if (t->total_rows == 0 || (!pool_row && !delta)) return IRM_OK;
  const uint32_t n = (uint32_t)t->total_rows;
  hipLaunchKernelGGL(gather_index_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), image_of(t), n, pool_row, delta);
  return launch_check("irm_table_gather_index");
}

extern "C" irm_status irm_rotate_gather(const irm_table* t, const void* pool, uint64_t pool_rows,
                                        void* out_kv, float* kr_f32, void* stream) {
  irm_status st = need_uploaded(t, "irm_rotate_gather");
  if (st != IRM_OK) return st;
  if (t->total_rows == 0) return IRM_OK;
  if ((st = check_pool(t, pool, pool_rows, "irm_rotate_gather")) != IRM_OK) return st;
  if (!out_kv || !aligned16(out_kv)) return fail(IRM_EINVAL, "irm_rotate_gather: out_kv NULL or misaligned");
  if (kr_f32 && !aligned16(kr_f32)) return fail(IRM_EINVAL, "irm_rotate_gather: kr_f32 misaligned");
  const uint32_t n = (uint32_t)t->total_rows;
  hipLaunchKernelGGL(rotate_gather_kernel, dim3((n + kTile - 1) / kTile), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), image_of(t), n,
                     static_cast<const uint4*>(pool), static_cast<uint4*>(out_kv), kr_f32);
  return launch_check("irm_rotate_gather");
}

extern "C" irm_status irm_mla_decode_workspace(const irm_table* t, uint32_t n_heads, uint32_t n_splits,
                                               size_t* bytes) {
  if (!t || !bytes) return fail(IRM_EINVAL, "irm_mla_decode_workspace: NULL argument");
  irm_status st = check_heads(n_heads, "irm_mla_decode_workspace");
  if (st != IRM_OK) return st;
  const uint32_t S = n_splits ? n_splits : default_splits(t, (n_heads / 16) / heads_per_block(n_heads / 16));
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
  const uint32_t S = n_splits ? n_splits : default_splits(t, G / heads_per_block(G));
  size_t need = 0;
  irm_mla_decode_workspace(t, n_heads, S, &need);
  if (!workspace || ws_bytes < need || reinterpret_cast<uintptr_t>(workspace) % irm::kAlign)
    return fail(IRM_EWORKSPACE, "irm_mla_decode: workspace missing, misaligned or smaller than "
                                "irm_mla_decode_workspace");
  const size_t parts = (size_t)t->n_seq * S * n_heads;
  if ((st = check_device()) != IRM_OK) return st;
  DecodeArgs a;
  a.im = image_of(t);
  a.pool = static_cast<const uint4*>(pool);
  a.q_lat = static_cast<const uint4*>(q_latent);
  a.q_rope = static_cast<const uint4*>(q_rope);
  a.ws_acc = static_cast<float*>(workspace);
  a.ws_ml = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) +
                                     irm::align_up(parts * IRM_D_LATENT * sizeof(float)));
  a.n_seq = t->n_seq;
  a.n_heads = n_heads;
  a.n_splits = S;
  a.pool_last = (uint32_t)((pool_rows < 0x100000000ull ? pool_rows : 0x100000000ull) - 1);
  a.scale_log2 = scale * kLog2e;
  // head groups per workgroup: 1 (4 column slices), 2 (2 slices) or 4 (full rows)
  const int hg = (int)heads_per_block(G);
  a.n_gblocks = G / hg;
  const uint64_t bs = (uint64_t)t->n_seq * S;
  const uint64_t grid = (bs + 7) / 8 * 8 * a.n_gblocks;
  if (grid > 0x7fffffffull) return fail(IRM_EUNSUPPORTED, "irm_mla_decode: grid too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hg == 4)
    hipLaunchKernelGGL((decode_split_kernel<4, 1, kDecodeDepth>), dim3((uint32_t)grid), dim3(kThreads), 0, s, a);
  else if (hg == 2)
    hipLaunchKernelGGL((decode_split_kernel<2, 2, kDecodeDepth>), dim3((uint32_t)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<1, 4, kDecodeDepth>), dim3((uint32_t)grid), dim3(kThreads), 0, s, a);
  if ((st = launch_check("irm_mla_decode: split kernel")) != IRM_OK) return st;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(t->n_seq * n_heads), dim3(128), 0, s, a.ws_acc, a.ws_ml,
                     static_cast<uint16_t*>(out), lse, n_heads, S);
  return launch_check("irm_mla_decode: combine kernel");
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
  PrefillArgs a;
  a.im = image_of(t);
  a.pool = static_cast<const uint4*>(pool);
  a.q_lat = static_cast<const uint4*>(q_latent);
  a.q_rope = static_cast<const uint4*>(q_rope);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.n_q = n_q;
  a.n_heads = n_heads;
  a.pool_last = (uint32_t)((pool_rows < 0x100000000ull ? pool_rows : 0x100000000ull) - 1);
  a.n_groups = n_heads / 16;
  a.q_pos0 = q_pos0;
  a.scale_log2 = scale * kLog2e;
  const uint64_t grid = (uint64_t)(n_q + 3) / 4 * a.n_groups;
  if (grid > 0x7fffffffull) return fail(IRM_EUNSUPPORTED, "irm_mla_prefill_tail: grid too large");
  hipLaunchKernelGGL(prefill_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream), a);
  return launch_check("irm_mla_prefill_tail");
}
