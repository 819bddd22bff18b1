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
  const uint4* rowmap;  // {pool row, delta, entry or kNoRot, 0} per assembled row
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
  im.rowmap = reinterpret_cast<const uint4*>(d + t->layout.off_rowmap);
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

// One rotation pair: (x, y) packed as bf16 in w, (cos, sin) = (c, s).
__device__ __forceinline__ uint32_t rotate_pair(uint32_t w, float c, float s) {
  const float x = bf16_lo(w), y = bf16_hi(w);
  return pack_bf16(fmaf(x, c, -(y * s)), fmaf(x, s, y * c));
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

// ---------------------------------------------------------------------------
// HBM -> LDS copies
//
// global_load_lds_dwordx4 moves 16 bytes per lane straight into LDS (lane l
// of a wave writes LDS address M0 + 16 l), so no registers hold data in
// flight.  The copies are issued from inline assembly and awaited with
// explicit s_waitcnt vmcnt; code between issue and wait must not touch
// global memory or scratch, since a wait the compiler inserts for such an
// access would also wait for every copy in flight.
//
// Stage layout: c_KV [rows][1024 B] then k_r [rows][128 B].  Within a row,
// 16-byte unit c of c_KV sits at position c ^ (r & 15) and unit u of k_r at
// u ^ ((r >> 1) & 7), so that 16 lanes reading the same unit of 16
// consecutive rows hit 16 different bank groups.
// ---------------------------------------------------------------------------
constexpr int kCkvBytes = IRM_D_LATENT * 2;  // 1024
constexpr int kKrBytes = IRM_D_ROPE * 2;     // 128

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

// A value the compiler must treat as freshly computed: keeps cheap per-lane
// index math inside the tile loop instead of hoisting dozens of addresses.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Wave-wide copy: lane l's 16 bytes at g land at LDS address lds + 16 l
// (one wait state between the M0 write and the LDS-DMA load).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "m0");
}

__device__ __forceinline__ void wait_dma_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t kr_pos(uint32_t r, uint32_t u) {
  return r * kKrBytes + ((u ^ ((r >> 1) & 7)) << 4);
}

struct StreamArgs {
  const unsigned char* pool;
  const uint4* rowmap;  // padded by kTile records past the last row
  uint32_t pool_last;
};

// ---------------------------------------------------------------------------
// MFMA building blocks on an LDS stage
//
// S^T for a 16-row block is K Q^T on v_mfma_f32_16x16x32_bf16: lane
// (q = lane/16, r = lane%16) gets the scores of rows row0 + 4q + i (i = 0..3)
// for head r.  O^T = C^T P^T then leaves every lane with outputs of a single
// head, so the online-softmax rescale is lane-local.  C^T operands come from
// transposing LDS reads (ds_read_b64_tr_b16): within each 16-lane group, lane
// 4a+b receives element b of the 8-byte reads of lanes a, a+4, a+8, a+12, so
// lane (q, s) reads row R0 + 4q + s/4, columns n0 + 4(s%4)..+3 and receives
// C[R0 + 4q + i][n0 + s], i = 0..3.  Softmax runs in the base-2 domain.
// ---------------------------------------------------------------------------

// Q^T operands of 16 heads for one query: lane (q, r) holds head head0 + r,
// dims 32 kk + 8 q .. +8 (kk 0..15 latent, 16..17 rope).
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
  // Consume the loads here: the tile loop below issues LDS copies the
  // compiler cannot see, and a wait for these loads inside the loop would
  // also wait for those copies.
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) asm volatile("" : "+a"(qb[kk]));
}

// Scores of NB 16-row blocks starting at row0 (a multiple of 16), blocks
// interleaved so that LDS reads overlap independent MFMAs.  Lane (q, rr)
// reads c_KV unit 4kk + q of row row0 + 16j + rr, stored at position
// (4kk + q) ^ rr = 4 (kk ^ (rr >> 2)) + (q ^ (rr & 3)): four per-lane bases
// (kk mod 4) plus an immediate 256 (kk / 4).
template <int NB>
__device__ __forceinline__ void qk_blocks(const unsigned char* ckv, const unsigned char* kr, uint32_t row0,
                                          const bf16x8_t (&qb)[18], f32x4_t (&acc)[NB]) {
  const uint32_t lane = opaque(threadIdx.x & 63), q = lane >> 4, rr = lane & 15;
  const unsigned char* rowp = ckv + (row0 + rr) * kCkvBytes + ((q ^ (rr & 3)) << 4);
  const unsigned char* base[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) base[i] = rowp + (((uint32_t)i ^ (rr >> 2)) << 6);
  const unsigned char* krp[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) krp[i] = kr + kr_pos(row0 + rr, 4 * i + q);
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    bf16x8_t a[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const unsigned char* ptr = kk < 16 ? base[kk & 3] + 256 * (kk >> 2) + 16 * j * kCkvBytes
                                         : krp[kk - 16] + 16 * j * kKrBytes;
      a[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(ptr));
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], qb[kk], acc[j], 0, 0, 0);
  }
}

typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4_ptr;

// Transposing reads of C^T for rows R0 + 4q + 0..3 (lane (q, s)), R0 a
// multiple of 16.  Lane (q, s) reads row R0 + 4q + s/4, 8 bytes at column
// 16 nb + 4 (s % 4): unit 2 nb + h (h = (s % 4) / 2), stored at position
// (2 nb + h) ^ x with x = (4q + s/4) = 2 (nb ^ (x >> 1)) + (h ^ (x & 1)), so
// eight per-lane bases (nb mod 8) plus an immediate 256 (nb / 8).
struct CtBases {
  const unsigned char* b[8];
};

__device__ __forceinline__ CtBases ct_bases(const unsigned char* st, uint32_t R0) {
  const uint32_t lane = opaque(threadIdx.x & 63), q = lane >> 4, s = lane & 15;
  const uint32_t x = 4 * q + (s >> 2);
  const uint32_t h = (s & 3) >> 1;
  const unsigned char* rowp = st + (R0 + x) * kCkvBytes + (((h ^ (x & 1))) << 4) + 8 * (s & 1);
  CtBases cb;
#pragma unroll
  for (int i = 0; i < 8; ++i) cb.b[i] = rowp + (((uint32_t)i ^ (x >> 1)) << 5);
  return cb;
}

__device__ __forceinline__ i16x4_t ct_read(const CtBases& cb, uint32_t nb) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(cb.b[nb & 7] + 256 * (nb >> 3)));
}

// O^T += C^T P^T over one 16-row block (k = 16) for 16-column blocks [nb0, nb0+NO).
template <int NO>
__device__ __forceinline__ void pv_block16(const unsigned char* st, uint32_t row0, uint32_t nb0, i16x4_t pb,
                                           f32x4_t (&o)[NO]) {
  const CtBases cb = ct_bases(st, row0);
  // all reads first: the MFMAs then run back to back while later reads land
  i16x4_t v[NO];
#pragma unroll
  for (int nb = 0; nb < NO; ++nb) v[nb] = ct_read(cb, nb0 + nb);
#pragma unroll
  for (int nb = 0; nb < NO; ++nb) o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v[nb], pb, o[nb], 0, 0, 0);
}

// Online softmax for one head per lane over NB blocks of 4 base-2 scores
// (-inf where masked): updates m and the lane-local partial sum l, rescales o
// when the maximum moved, and leaves the probabilities in p.
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

__device__ __forceinline__ i16x4_t pack_p4(const float (&a)[4]) {
  const uint2 w = make_uint2(pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]));
  return __builtin_bit_cast(i16x4_t, w);
}

__device__ __forceinline__ bf16x8_t pack_p8(const float (&a)[4], const float (&b)[4]) {
  const uint4 w = make_uint4(pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]),
                             pack_bf16(b[2], b[3]));
  return __builtin_bit_cast(bf16x8_t, w);
}

__device__ __forceinline__ void fill_omega(double* omega, const InvFreq& f) {
  if (threadIdx.x < irm::kPairs) omega[threadIdx.x] = f.w[threadIdx.x];
}

// ---------------------------------------------------------------------------
// split-KV decode, pass 1: wave-private KV streams
//
// Workgroup = (sequence, split, 16-head group), 4 waves, one workgroup per
// CU.  The split's rows are cut into four contiguous ranges, one per wave,
// and every wave streams its range on its own: 16-row tiles are copied
// HBM -> LDS into a private two-stage ring (global_load_lds_dwordx4), k_r is
// rotated in place, and the wave scores the 16 rows for its 16 heads and
// accumulates all 512 output columns.  Nothing in the tile loop waits for
// another wave; the four online-softmax states merge once at the end.
//
// Per iteration t a wave issues the row map of tile t+3 (one copy) and the
// data of tile t+1 (16 c_KV rows + 2 k_r copies), then waits until at most
// those 19 copies are outstanding, which means tile t has landed.
// ---------------------------------------------------------------------------
constexpr int kWaveRows = 16;
constexpr int kWaveRm = 4;                                          // row-map slots
constexpr int kWaveStageKr = kWaveRows * kCkvBytes;                 // k_r region of a stage
constexpr int kWaveStageBytes = kWaveRows * (kCkvBytes + kKrBytes); // 18432
constexpr int kWaveCopies = 1 + kWaveRows + 2;                      // copies per iteration

struct WaveRing {
  unsigned char stage[2][kWaveStageBytes];
  uint4 rm[kWaveRm][kWaveRows];  // row-map records
  float2 trig[2][irm::kPairs];   // (cos, sin) for two deltas
};

struct DecodeSmem {
  WaveRing w[kThreads / 64];
  double omega[irm::kPairs];
  float ml[kThreads / 64][16][2];
};

__device__ __forceinline__ void wave_wait_tile() { asm volatile("s_waitcnt vmcnt(19)" ::: "memory"); }
__device__ __forceinline__ void wave_wait_rm() { asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); }
static_assert(kWaveCopies == 19, "the wave wait counts one iteration's copies");

struct WaveRange {
  uint32_t g_begin, n, ntiles;
  __device__ uint32_t g0(uint32_t x) const { return g_begin + min(x, ntiles - 1) * kWaveRows; }
};

// Row map of tile x (16 records of 16 B, one per lane 0..15); x is clamped to the last tile.
__device__ __forceinline__ void wave_issue_rowmap(const StreamArgs& ra, const WaveRange& wr, WaveRing& wv, uint32_t x) {
  const uint32_t l = threadIdx.x & 63;
  if (l < kWaveRows) dma16(ra.rowmap + wr.g0(x) + l, lds_addr(&wv.rm[x % kWaveRm][0]));
}

// Data of tile x: one 1 KB c_KV row per copy, then k_r of rows 0-7 and 8-15.
// Pool rows are clamped so that a corrupted map yields wrong values, not a fault.
__device__ __forceinline__ void wave_issue_data(const StreamArgs& ra, WaveRing& wv, uint32_t x) {
  const uint32_t l = opaque(threadIdx.x & 63);
  unsigned char* st = wv.stage[x & 1];
  const uint4* rec = wv.rm[x % kWaveRm];
  uint32_t src[kWaveRows];
#pragma unroll
  for (int r = 0; r < kWaveRows; ++r) src[r] = min(rec[r].x, ra.pool_last);
  const uint32_t kr0 = min(rec[l >> 3].x, ra.pool_last), kr1 = min(rec[8 + (l >> 3)].x, ra.pool_last);
#pragma unroll
  for (int r = 0; r < kWaveRows; ++r)
    dma16(ra.pool + (size_t)src[r] * kRowBytes + ((l ^ r) << 4), lds_addr(st + r * kCkvBytes));
  const uint32_t r0 = l >> 3, r1 = 8 + (l >> 3);
  dma16(ra.pool + (size_t)kr0 * kRowBytes + kCkvBytes + (((l & 7) ^ ((r0 >> 1) & 7)) << 4),
        lds_addr(st + kWaveStageKr));
  dma16(ra.pool + (size_t)kr1 * kRowBytes + kCkvBytes + (((l & 7) ^ ((r1 >> 1) & 7)) << 4),
        lds_addr(st + kWaveStageKr + 8 * kKrBytes));
}

// Rotate the k_r of a landed tile in place.  Lane l handles row l/4 and the
// logical k_r units 2 (l%4) and 2 (l%4) + 1, i.e. pairs 8 (l%4) .. +7.  The
// wave keeps (cos, sin) of all 32 pairs for two deltas in LDS (cd[0], cd[1];
// 0 marks an empty slot, delta 0 needs no rotation).  Rows whose delta is in
// the table rotate at once; otherwise a round evaluates the table for two of
// the missing deltas (those of the first and the last lane still waiting).
// Deltas change only at entry boundaries, so most tiles need no round.
__device__ __forceinline__ void wave_rotate(WaveRing& wv, unsigned char* st, const double* omega, int32_t d,
                                            int32_t (&cd)[2]) {
  const uint32_t l = threadIdx.x & 63, r = l >> 2, u0 = 2 * (l & 3);
  bool todo = d != 0;
  while (__any(todo)) {
    if (todo && (d == cd[0] || d == cd[1])) {
      const f32x4_t* tp = reinterpret_cast<const f32x4_t*>(&wv.trig[d == cd[0] ? 0 : 1][8 * (l & 3)]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4_t a = tp[2 * h], b = tp[2 * h + 1];
        u32x4_t* p = reinterpret_cast<u32x4_t*>(st + kWaveStageKr + kr_pos(r, u0 + h));
        const u32x4_t k = *p;
        const u32x4_t o = {rotate_pair(k[0], a[0], a[1]), rotate_pair(k[1], a[2], a[3]),
                           rotate_pair(k[2], b[0], b[1]), rotate_pair(k[3], b[2], b[3])};
        *p = o;
      }
      todo = false;
    }
    const uint64_t mask = __ballot(todo);
    if (mask == 0) break;
    cd[0] = __shfl(d, __ffsll((unsigned long long)mask) - 1);
    cd[1] = __shfl(d, 63 - __clzll((long long)mask));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // every lane is done with the old table
    {
      double sn, cn;
      sincos((double)cd[l >> 5] * omega[l & 31], &sn, &cn);
      wv.trig[l >> 5][l & 31] = make_float2((float)cn, (float)sn);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

struct DecodeArgs {
  StreamArgs ra;
  const uint32_t* seq_base;
  const uint4* q_lat;
  const uint4* q_rope;
  float* ws_acc;  // [n_seq][n_splits][n_heads][512], unnormalised
  float* ws_ml;   // [n_seq][n_splits][n_heads][2]: base-2 max, sum
  uint32_t n_seq, n_heads, n_groups, n_splits;
  float scale_log2;
  InvFreq f;
};

__global__ __launch_bounds__(kThreads, 1) void decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) DecodeSmem sm;

  // Workgroups of the same (sequence, split) but different head groups get
  // the same x % 8, i.e. the same XCD and L2, at consecutive slots.
  const uint32_t x = blockIdx.x, xcd = x & 7, slot = x >> 3;
  const uint32_t g = slot % a.n_groups;
  const uint32_t bs = (slot / a.n_groups) * 8 + xcd;
  if (bs >= a.n_seq * a.n_splits) return;
  const uint32_t b = bs / a.n_splits, sp = bs % a.n_splits;

  const uint32_t base = a.seq_base[b];
  const uint32_t N = a.seq_base[b + 1] - base;
  const uint32_t per = ((N + a.n_splits - 1) / a.n_splits + 63) / 64 * 64;
  const uint32_t r0 = min(N, sp * per), r1 = min(N, r0 + per);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hq = lane >> 4, hr = lane & 15;
  const uint32_t head = g * 16 + hr;

  // this wave's rows: a quarter of the split, in whole tiles
  const uint32_t quarter = ((r1 - r0 + 3) / 4 + kWaveRows - 1) / kWaveRows * kWaveRows;
  const uint32_t w0 = min(r1, r0 + wave * quarter), w1 = min(r1, w0 + quarter);
  WaveRange wr;
  wr.g_begin = base + w0;
  wr.n = w1 - w0;
  wr.ntiles = (wr.n + kWaveRows - 1) / kWaveRows;
  WaveRing& wv = sm.w[wave];

  bf16x8_t qb[18];
  load_q(a.q_lat, a.q_rope, b, a.n_heads, head, qb);
  fill_omega(sm.omega, a.f);
  f32x4_t o[32];
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  int32_t cd[2] = {0, 0};  // deltas held in the wave's trig table
  __syncthreads();

  if (wr.ntiles > 0) {
    for (uint32_t t = 0; t < 3; ++t) wave_issue_rowmap(a.ra, wr, wv, t);
    wait_dma_all();
    wave_issue_data(a.ra, wv, 0);
    for (uint32_t t = 0; t < wr.ntiles; ++t) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of the stage about to be refilled are done
      wave_issue_rowmap(a.ra, wr, wv, t + 3);
      if (t + 1 < wr.ntiles) {
        wave_issue_data(a.ra, wv, t + 1);
        wave_wait_tile();
      } else {
        wave_wait_rm();
      }
      unsigned char* st = wv.stage[t & 1];
      const uint32_t nrows = min((uint32_t)kWaveRows, wr.n - t * kWaveRows);
      const int32_t d = (int32_t)wv.rm[t % kWaveRm][lane >> 2].y;
      wave_rotate(wv, st, sm.omega, d, cd);
      f32x4_t acc[1];
      qk_blocks<1>(st, st + kWaveStageKr, 0, qb, acc);
      float sc[1][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[0][i] = (4 * hq + i < (int)nrows) ? acc[0][i] * a.scale_log2 : -INFINITY;
      float p[1][4];
      softmax_update_n<1, 32>(sc, m, l, o, p);
      pv_block16<32>(st, 0, 0, pack_p4(p[0]), o);
    }
    wait_dma_all();  // the last row-map copies
  }

  // merge the four waves' softmax states
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (hq == 0) {
    sm.ml[wave][hr][0] = m;
    sm.ml[wave][hr][1] = l;
  }
  __syncthreads();
  float mstar = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) mstar = fmaxf(mstar, sm.ml[w][hr][0]);
  float lsum = 0.f, fw = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = sm.ml[w][hr][0];
    const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - mstar);
    lsum += sm.ml[w][hr][1] * f;
    if (w == wave) fw = f;
  }
  float* red = reinterpret_cast<float*>(&sm.w[0].stage[0][0]);  // [4 waves][16 heads][512]
  static_assert(4 * 16 * IRM_D_LATENT * 4 <= 4 * sizeof(WaveRing), "merge buffer fits the rings");
  float* mine = red + wave * 16 * IRM_D_LATENT;
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) {
    float4 v = make_float4(fw * o[nb][0], fw * o[nb][1], fw * o[nb][2], fw * o[nb][3]);
    *reinterpret_cast<float4*>(mine + hr * IRM_D_LATENT + 16 * nb + 4 * hq) = v;
  }
  __syncthreads();
  const size_t pidx = ((size_t)b * a.n_splits + sp) * a.n_heads + g * 16;
  float4* dst = reinterpret_cast<float4*>(a.ws_acc + pidx * IRM_D_LATENT);
  const float4* src = reinterpret_cast<const float4*>(red);
  constexpr int kQuads = 16 * IRM_D_LATENT / 4;
  for (int i = threadIdx.x; i < kQuads; i += kThreads) {
    const float4 v0 = src[i], v1 = src[i + kQuads], v2 = src[i + 2 * kQuads], v3 = src[i + 3 * kQuads];
    dst[i] = make_float4(v0.x + v1.x + v2.x + v3.x, v0.y + v1.y + v2.y + v3.y, v0.z + v1.z + v2.z + v3.z,
                         v0.w + v1.w + v2.w + v3.w);
  }
  if (threadIdx.x < 16) {
    a.ws_ml[(pidx + threadIdx.x) * 2 + 0] = mstar;
    a.ws_ml[(pidx + threadIdx.x) * 2 + 1] = (mstar == -INFINITY) ? 0.f : lsum;
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

uint32_t default_splits(const irm_table* t, uint32_t n_groups) {
  // one workgroup per CU (256 CUs) with >= 256 rows per split
  const uint32_t want = (256 + t->n_seq * n_groups - 1) / (t->n_seq * n_groups);
  const uint32_t cap = (t->max_seq_len + 255) / 256;
  uint32_t s = want < cap ? want : cap;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return s;
}

// Last pool row a kernel may touch (pool_rows is clamped to 2^32).
uint32_t pool_last_of(uint64_t pool_rows) {
  return (uint32_t)((pool_rows < 0x100000000ull ? pool_rows : 0x100000000ull) - 1);
}

StreamArgs stream_args(const irm_table* t, const void* pool, uint64_t pool_rows) {
  StreamArgs ra;
  ra.pool = static_cast<const unsigned char*>(pool);
  ra.rowmap = image_of(t).rowmap;
  ra.pool_last = pool_last_of(pool_rows);
  return ra;
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
  {
    const uint32_t n = (uint32_t)t->total_rows;
    const Image im = image_of(t);
    hipLaunchKernelGGL(rowmap_kernel, dim3((n + kTile + 255) / 256), dim3(256), 0, s, im, n,
                       const_cast<uint4*>(im.rowmap));
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
  std::memcpy(t->inv_freq, inv_freq, sizeof(t->inv_freq));
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
  const uint32_t S = n_splits ? n_splits : default_splits(t, n_heads / 16);
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
  const uint32_t S = n_splits ? n_splits : default_splits(t, G);
  size_t need = 0;
  irm_mla_decode_workspace(t, n_heads, S, &need);
  if (!workspace || ws_bytes < need || reinterpret_cast<uintptr_t>(workspace) % irm::kAlign)
    return fail(IRM_EWORKSPACE, "irm_mla_decode: workspace missing, misaligned or smaller than "
                                "irm_mla_decode_workspace");
  const size_t parts = (size_t)t->n_seq * S * n_heads;
  if ((st = check_device()) != IRM_OK) return st;
  DecodeArgs a;
  a.ra = stream_args(t, pool, pool_rows);
  a.seq_base = image_of(t).seq_base;
  a.q_lat = static_cast<const uint4*>(q_latent);
  a.q_rope = static_cast<const uint4*>(q_rope);
  a.ws_acc = static_cast<float*>(workspace);
  a.ws_ml = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) +
                                     irm::align_up(parts * IRM_D_LATENT * sizeof(float)));
  a.n_seq = t->n_seq;
  a.n_heads = n_heads;
  a.n_groups = G;
  a.n_splits = S;
  a.scale_log2 = scale * kLog2e;
  std::memcpy(a.f.w, t->inv_freq, sizeof(a.f.w));
  const uint64_t bs = (uint64_t)t->n_seq * S;
  const uint64_t grid = (bs + 7) / 8 * 8 * G;
  if (grid > 0x7fffffffull) return fail(IRM_EUNSUPPORTED, "irm_mla_decode: grid too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(decode_split_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, s, a);
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
  a.pool_last = pool_last_of(pool_rows);
  a.n_groups = n_heads / 16;
  a.q_pos0 = q_pos0;
  a.scale_log2 = scale * kLog2e;
  const uint64_t grid = (uint64_t)(n_q + 3) / 4 * a.n_groups;
  if (grid > 0x7fffffffull) return fail(IRM_EUNSUPPORTED, "irm_mla_prefill_tail: grid too large");
  hipLaunchKernelGGL(prefill_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream), a);
  return launch_check("irm_mla_prefill_tail");
}
