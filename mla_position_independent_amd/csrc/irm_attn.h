// Device building blocks shared by the attention kernels: HBM -> LDS copies
// and the MFMA score / value products with the online softmax.
//
// Absorbed MLA attention (Irminsul pages: gentlecold.top article, section 4):
// score = q_lat . c_KV + q_rope . k_r over the 576-wide row, value = c_KV.
#pragma once

#include <type_traits>

#include "irm_device.h"

namespace irm {
namespace dev {

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

// Wave-wide copy: lane l's 16 bytes at g land at LDS address lds + 16 l.
// The compiler writes M0 (an input operand of the asm) right before it; the
// s_nop gives the one wait state between that write and the LDS-DMA load.
// kStream marks data read exactly once (the non-temporal policy keeps it
// from displacing rows that other workgroups still read from the caches).
template <bool kStream = false>
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  if constexpr (kStream)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(g), "{m0}"(m0));
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(m0));
}

// The same copy from base + off, base the same for every lane (scalar
// registers, so its 64-bit address math is scalar) and off a 32-bit per-lane
// offset: the form for copies of one row, whose source is wave-uniform.
template <bool kStream = false>
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  if constexpr (kStream)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(off), "s"(base), "{m0}"(m0));
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(m0));
}

__device__ __forceinline__ void wait_dma_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t kr_pos(uint32_t r, uint32_t u) {
  return r * kKrBytes + ((u ^ ((r >> 1) & 7)) << 4);
}

struct StreamArgs {
  const unsigned char* pool;
  const uint4* rowmap;  // padded by kTile records past the last row
  const float2* trig;   // (cos, sin) of every entry's delta, [n_entries][32]
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
template <bool kInAgpr = true>
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
  // Consume the loads here: the tile loop issues LDS copies the compiler
  // cannot see, and a wait for these loads inside the loop would also wait
  // for those copies.  The operands then stay in the register file asked for
  // (MFMA reads its B operand from either).
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    if constexpr (kInAgpr)
      asm volatile("" : "+a"(qb[kk]));
    else
      asm volatile("" : "+v"(qb[kk]));
  }
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
  auto read = [&](int kk, bf16x8_t (&a)[NB]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const unsigned char* ptr = kk < 16 ? base[kk & 3] + 256 * (kk >> 2) + 16 * j * kCkvBytes
                                         : krp[kk - 16] + 16 * j * kKrBytes;
      a[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(ptr));
    }
  };
  // double-buffered: the reads of step kk+1 are in flight while step kk's MFMAs run
  bf16x8_t cur[NB], nxt[NB];
  read(0, cur);
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    if (kk + 1 < 18) read(kk + 1, nxt);
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur[j], qb[kk], acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NB; ++j) cur[j] = nxt[j];
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

// O^T += C^T P^T over a pair of 16-row blocks (rows row0.. and row0+16..) on
// v_mfma_f32_16x16x32_bf16; the k order {4q..4q+3, 16+4q..16+4q+3} matches
// the lane's probabilities of the two blocks, packed in pb.  Reads go out in
// groups of eight column blocks, each group ahead of its MFMAs.
template <int NO>
__device__ __forceinline__ void pv_pair(const unsigned char* st, uint32_t row0, uint32_t nb0, bf16x8_t pb,
                                        f32x4_t (&o)[NO]) {
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const CtBases c0 = ct_bases(st, row0);
  constexpr int kGroup = NO < 8 ? NO : 8;
#pragma unroll
  for (int g0 = 0; g0 < NO; g0 += kGroup) {
    i16x8_t v[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int nb = nb0 + g0 + j;
      const i16x4_t lo = ct_read(c0, nb);
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_ptr)(c0.b[nb & 7] + 256 * (nb >> 3) + 16 * kCkvBytes));
      v[j] = i16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j)
      o[g0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v[j]), pb, o[g0 + j], 0, 0, 0);
  }
}

// Online softmax for one head per lane over NB blocks of 4 raw scores (-inf
// where masked), in the base-2 domain: p = 2^(s c - m) with c = scale log2(e).
// m is a reference maximum that moves only when a score exceeds it by more
// than kSlack (or on the first finite score), so most tiles skip the rescale
// of o; p then stays below 2^kSlack, harmless in bf16 and in the float sums.
// Updates m, the lane-local partial sum l and o, and leaves p.
constexpr float kSlack = 8.f;

template <int NB, int NO>
__device__ __forceinline__ void softmax_update_n(const float (&s)[NB][4], float c, float& m, float& l,
                                                 f32x4_t (&o)[NO], float (&p)[NB][4]) {
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[j][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mxc = mx * c;  // -inf stays -inf (c > 0)
  if (__any(mxc > m + kSlack)) {  // m == -inf takes this path on the first finite score
    const float m_new = (mxc > m + kSlack) ? mxc : m;
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 1 if unchanged, 0 from -inf
    l *= alpha;
#pragma unroll
    for (int nb = 0; nb < NO; ++nb) o[nb] *= alpha;
    m = m_new;
  }
  const float m_use = (m == -INFINITY) ? 0.f : m;
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[j][i] = __builtin_amdgcn_exp2f(fmaf(s[j][i], c, -m_use));
      sum += p[j][i];
    }
  l += sum;
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
// Slices: R consecutive rows (R = 8 or 16) that one wave copies HBM -> LDS on
// its own, placed at tile rows row0 .. row0+R-1 of a stage (the unit swizzle
// depends on the tile row).  Per slice a wave issues one row-map copy (R
// records of 16 B, lanes 0..R-1) and R + R/8 data copies (one 1 KB c_KV row
// each, then the k_r of 8 rows per copy).
// ---------------------------------------------------------------------------
template <int kSlots, int R>
struct WaveSlots {
  uint4 rm[kSlots][R];     // row-map records of prefetched slices
  float2 trig[2][kPairs];  // (cos, sin) of all pairs for two deltas
};

// Row map of the slice whose first assembled row is g0, into rm.
template <int R>
__device__ __forceinline__ void slice_issue_rowmap(const StreamArgs& ra, uint32_t g0, uint4* rm) {
  const uint32_t l = threadIdx.x & 63;
  if (l < (uint32_t)R) dma16s(ra.rowmap + (uint32_t)__builtin_amdgcn_readfirstlane(g0), 16 * l, lds_addr(rm));
}

// Start of pool row src (wave-uniform) as a scalar address.
__device__ __forceinline__ const unsigned char* pool_row(const StreamArgs& ra, uint32_t src) {
  return ra.pool + (size_t)(uint32_t)__builtin_amdgcn_readfirstlane(src) * kRowBytes;
}

// Data of the slice described by rec into tile rows row0.. of the stage with
// c_KV at ckv and k_r at kr, streamed (every row is read once per launch by
// the workgroup that copies it).  Pool rows are clamped so that a corrupted
// map yields wrong values, never a fault.
template <int R>
__device__ __forceinline__ void slice_issue_data(const StreamArgs& ra, const uint4* rec, unsigned char* ckv,
                                                 unsigned char* kr, uint32_t row0) {
  const uint32_t l = opaque(threadIdx.x & 63);
  uint32_t src[R];
#pragma unroll
  for (int k = 0; k < R; ++k) src[k] = min(rec[k].x, ra.pool_last);
  uint32_t ksrc[R / 8];
#pragma unroll
  for (int h = 0; h < R / 8; ++h) ksrc[h] = min(rec[8 * h + (l >> 3)].x, ra.pool_last);
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const uint32_t r = row0 + k;
    dma16s<true>(pool_row(ra, src[k]), (l ^ (r & 15)) << 4, lds_addr(ckv + r * kCkvBytes));
  }
#pragma unroll
  for (int h = 0; h < R / 8; ++h) {
    const uint32_t r = row0 + 8 * h + (l >> 3);
    dma16<true>(ra.pool + (size_t)ksrc[h] * kRowBytes + kCkvBytes + (((l & 7) ^ ((r >> 1) & 7)) << 4),
                lds_addr(kr + (row0 + 8 * h) * kKrBytes));
  }
}

// Rotate the k_r of a landed slice in place.  Lane l handles slice row
// l / (64 / R) and R / 8 logical k_r units (4 pairs each); d is that row's
// delta.  The wave keeps (cos, sin) of all 32 pairs for two deltas in LDS
// (cd[0], cd[1]; 0 marks an empty slot, delta 0 needs no rotation).  Rows
// whose delta is in the table rotate at once; otherwise a round evaluates
// the table in double for two of the missing deltas (those of the first and
// the last lane still waiting).  Deltas change only at entry boundaries, so
// most slices need no round.  Nothing here touches global memory or scratch
// (see dma16).
template <int R, int kSlots>
__device__ __forceinline__ void slice_rotate(WaveSlots<kSlots, R>& ws, unsigned char* kr, uint32_t row0,
                                             const double* omega, int32_t d, int32_t (&cd)[2]) {
  constexpr int kUnits = R / 8;  // units per lane
  const uint32_t l = threadIdx.x & 63, r = row0 + l / (64 / R), u0 = kUnits * (l % (64 / R));
  bool todo = d != 0;
  while (__any(todo)) {
    if (todo && (d == cd[0] || d == cd[1])) {
      const f32x4_t* tp = reinterpret_cast<const f32x4_t*>(&ws.trig[d == cd[0] ? 0 : 1][4 * u0]);
#pragma unroll
      for (int h = 0; h < kUnits; ++h) {
        const f32x4_t a = tp[2 * h], b = tp[2 * h + 1];
        u32x4_t* p = reinterpret_cast<u32x4_t*>(kr + kr_pos(r, u0 + h));
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
      ws.trig[l >> 5][l & 31] = make_float2((float)cn, (float)sn);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Delta of the slice row that lane l rotates.
template <int R>
__device__ __forceinline__ int32_t slice_row_delta(const uint4* rec) {
  return (int32_t)rec[(threadIdx.x & 63) / (64 / R)].y;
}

// Fill the wave's trig table with the precomputed (cos, sin) rows of the
// entries of two slice rows, the first and the last with a nonzero delta
// (lane l holds delta d of its row, rec the slice's row-map records): lanes
// 0..15 copy the first entry's 256 bytes into slot 0, lanes 16..31 the last
// one's into slot 1, and cd takes the two deltas.  Does nothing when the
// table already holds every nonzero delta of the slice (most slices), so a
// copy goes out only at entry boundaries; callers' waits count only copies
// issued after it.
template <int kSlots, int R>
__device__ __forceinline__ void slice_trig_fetch(const StreamArgs& ra, WaveSlots<kSlots, R>& ws, int32_t d,
                                                 const uint4* rec, int32_t (&cd)[2]) {
  if (!__any(d != 0 && d != cd[0] && d != cd[1])) return;
  const uint32_t l = threadIdx.x & 63;
  const uint64_t nz = __ballot(d != 0);
  const int first = __ffsll((unsigned long long)nz) - 1, last = 63 - __clzll((long long)nz);
  cd[0] = __shfl(d, first);
  cd[1] = __shfl(d, last);
  const uint32_t ent = rec[(uint32_t)((l < 16) ? first : last) / (64 / R)].z;
  if (l < 32) dma16(ra.trig + (size_t)ent * kPairs + 2 * (l & 15), lds_addr(&ws.trig[0][0]));
}

template <int N>
__device__ __forceinline__ void wait_dma_but() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// ---------------------------------------------------------------------------
// Shared 32-row tiles: four waves each copy and rotate one 8-row slice of
// every tile into a four-stage LDS ring, and all four compute on the whole
// tile.  A stage holds the tile's c_KV rows (1 KB each, 16-byte units
// swizzled by row) and then its k_r rows (128 B each).
// ---------------------------------------------------------------------------
constexpr int kTileRows = 32;
constexpr int kStages = 4;
constexpr int kTileSlice = kTileRows / 4;                       // rows per wave and tile
constexpr int kTileRm = 8;                                      // row-map slots per wave
constexpr int kTileKr = kTileRows * kCkvBytes;                  // k_r region of a stage
constexpr int kTileBytes = kTileRows * (kCkvBytes + kKrBytes);  // 36864

struct SharedSmem {
  unsigned char stage[kStages][kTileBytes];
  WaveSlots<kTileRm, kTileSlice> slots[4];
  double omega[kPairs];
};

// ---------------------------------------------------------------------------
// Split tiles: four groups of 16 query-heads per workgroup, output columns
// split across the accumulating waves
//
// Each 32-row tile serves four groups of 16 query-heads (four queries of one
// head group in prefill, four head groups of one query in decode).  Scoring
// wave s computes the scores of group s (K fragments from LDS, Q in
// registers), runs its online softmax, and publishes the probabilities
// (already in the lane layout of the PV B operand) and any rescale factors
// through LDS.  After a barrier, accumulating wave j sums O for all four
// groups over output columns 128 j .. 128 j + 127, so every C^T fragment it
// reads feeds four MFMAs.  Per tile and SIMD: 36 + 32 MFMAs; LDS reads 36 KB
// (K) + 8 KB (C^T) + 4 KB (P), against 36 KB + 32 KB when one wave
// accumulates all columns of its own group.
// ---------------------------------------------------------------------------
constexpr int kSplitGroups = 4;
constexpr int kSplitCols = IRM_D_LATENT / kSplitGroups;  // 128 output columns per wave
constexpr int kSplitNb = kSplitCols / 16;                // 8 column blocks

struct SplitSmem {
  SharedSmem s;
  // per tile parity: P of tile t is produced in iteration t and consumed in t+1
  uint4 pfrag[2][kSplitGroups][64];  // P^T operand of group g for lane l (8 bf16)
  float alpha[2][kSplitGroups][16];  // rescale factor of group g, head l % 16
  uint32_t scaled[2][kSplitGroups];  // group g moved its reference maximum on that tile
  float ml[kSplitGroups][16][2];     // final (m, l) of group g, head l % 16
};
static_assert(sizeof(SplitSmem) <= 160 * 1024, "split tiles fit the LDS");

// Maximum over the four lane quarters of a wave (lanes l, l^16, l^32, l^48),
// with the two permlane swaps: each gives every lane its own value and its
// partner's, in some order.
__device__ __forceinline__ float max_quarters(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Online softmax of one group over 2 blocks of 4 raw scores per lane (-inf
// where masked), without touching O and without branches: leaves p and
// alpha (1 where the head's reference maximum did not move), returns whether
// any head moved it.
__device__ __forceinline__ bool softmax_scores(const float (&s)[2][4], float c, float& m, float& l,
                                               float (&p)[2][4], float& alpha) {
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[j][i]);
  mx = max_quarters(mx);
  const float mxc = mx * c;
  const bool mv = mxc > m + kSlack;
  const float m_new = mv ? mxc : m;
  alpha = mv ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
  l *= alpha;
  m = m_new;
  const float m_use = (m == -INFINITY) ? 0.f : m;
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[j][i] = __builtin_amdgcn_exp2f(fmaf(s[j][i], c, -m_use));
      sum += p[j][i];
    }
  l += sum;
  return __any(mv);
}

// Scoring waves publish (m, l) of their group; after this every
// accumulating wave can normalise its columns of all four groups.  l is
// reduced over the lane quarters here.  The accumulating waves meet the
// barrier with split_publish_wait.
__device__ __forceinline__ void split_publish(SplitSmem& sm, float m, float l) {
  const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if ((lane >> 4) == 0) {
    sm.ml[w][lane & 15][0] = m;
    sm.ml[w][lane & 15][1] = l;
  }
  __syncthreads();
}

__device__ __forceinline__ void split_publish_wait() { __syncthreads(); }

// The copies of one wave's 8-row slice of a tile, prepared from its row-map
// records and issued one by one between the score MFMAs of the current tile.
struct SliceCopies {
  uint32_t src[kTileSlice];  // pool row of each c_KV row
  uint32_t ksrc;             // pool row of the k_r row this lane copies
};

__device__ __forceinline__ SliceCopies prep_copies(const StreamArgs& ra, const uint4* rec) {
  const uint32_t l = opaque(threadIdx.x & 63);
  SliceCopies cp;
#pragma unroll
  for (int k = 0; k < kTileSlice; ++k) cp.src[k] = min(rec[k].x, ra.pool_last);
  cp.ksrc = min(rec[l >> 3].x, ra.pool_last);
  return cp;
}

// c_KV row row0 + k of the slice into the stage at ckv (1 KB, one copy).
__device__ __forceinline__ void copy_ckv(const StreamArgs& ra, const SliceCopies& cp, int k, unsigned char* ckv,
                                         uint32_t row0) {
  const uint32_t l = threadIdx.x & 63, r = row0 + k;
  dma16s(pool_row(ra, cp.src[k]), (l ^ (r & 15)) << 4, lds_addr(ckv + r * kCkvBytes));
}

// k_r of the slice's 8 rows into the stage's k_r region (1 KB, one copy).
__device__ __forceinline__ void copy_kr(const StreamArgs& ra, const SliceCopies& cp, unsigned char* kr,
                                        uint32_t row0) {
  const uint32_t l = threadIdx.x & 63, r = row0 + (l >> 3);
  dma16(ra.pool + (size_t)cp.ksrc * kRowBytes + kCkvBytes + (((l & 7) ^ ((r >> 1) & 7)) << 4),
        lds_addr(kr + row0 * kKrBytes));
}

// Rotation of the slice's k_r from the table in two halves, so that the
// LDS read can be issued well before the arithmetic and the write: lane l
// turns unit l % 8 of row l / 8; rows with delta 0 take the identity (cos 1,
// sin 0).
struct SliceRot {
  u32x4_t k;
  f32x4_t a, b;
};

template <int kSlots>
__device__ __forceinline__ SliceRot slice_rot_load(const WaveSlots<kSlots, kTileSlice>& ws, const unsigned char* kr,
                                                   uint32_t row0, int32_t d, const int32_t (&cd)[2]) {
  const uint32_t l = threadIdx.x & 63, r = row0 + (l >> 3), u = l & 7;
  const f32x4_t* tp = reinterpret_cast<const f32x4_t*>(&ws.trig[d == cd[0] ? 0 : 1][4 * u]);
  SliceRot x;
  x.a = tp[0];
  x.b = tp[1];
  if (d == 0) {
    x.a = f32x4_t{1.f, 0.f, 1.f, 0.f};
    x.b = x.a;
  }
  x.k = *reinterpret_cast<const u32x4_t*>(kr + kr_pos(r, u));
  return x;
}

__device__ __forceinline__ void slice_rot_store(unsigned char* kr, uint32_t row0, const SliceRot& x) {
  const uint32_t l = threadIdx.x & 63, r = row0 + (l >> 3), u = l & 7;
  *reinterpret_cast<u32x4_t*>(kr + kr_pos(r, u)) =
      u32x4_t{rotate_pair(x.k[0], x.a[0], x.a[1]), rotate_pair(x.k[1], x.a[2], x.a[3]),
              rotate_pair(x.k[2], x.b[0], x.b[1]), rotate_pair(x.k[3], x.b[2], x.b[3])};
}

// ---------------------------------------------------------------------------
// Role-split streaming of split tiles: eight waves per workgroup, two per
// SIMD.  Waves 0..3 score: wave s holds Q of group s, computes S^T of every
// tile, runs the online softmax and publishes P and the rescale factors.
// Waves 4..7 accumulate: wave 4+j sums O of all four groups over output
// columns 128 j .. 128 j + 127.  Each SIMD thus runs one wave of each kind,
// and either covers the other's LDS, copy and barrier waits with its MFMAs.
// Slice j of a tile (rows 8j..8j+7) is copied by scorer j (its first
// kScoreRows c_KV rows) and accumulator j (the other c_KV rows, the k_r and
// the row maps), and rotated by accumulator j.
//
// Iteration t (0 <= t <= nt) ends with one barrier.  Scorers (t < nt):
// scores of tile t with their copies of tile t+2 between the MFMAs, softmax,
// P under parity t, then a wait for their copies of tile t+1.  Accumulators:
// wait for tile t+1 and rotate their slice of it, PV of tile t-1 (t >= 1)
// from the P published one iteration earlier with their copies of tile t+2
// between the MFMAs, the row map of tile t+4.  Stages in use during
// iteration t: t-1 (PV), t (QK), t+1 (rotate), t+2 (copies in flight).
// Copies of tiles past the end re-read the last tile into the free stage,
// so every iteration issues the same copies per wave and the waits count
// them.  Barriers per call: nt + 2 on both sides, none when nt = 0.
//
// Flat mode (kFlat): the rows are an assembled cache, row g of the stream is
// row g of the buffer and every delta is 0, so no row maps are copied and
// nothing is rotated.
// ---------------------------------------------------------------------------
constexpr int kRoleThreads = 2 * kThreads;
// c_KV rows of each slice that the scorer copies: all of them, since the
// accumulating waves (k_r, row maps, rotation, PV) are the longer chain
// when rows come through the chunk table (about 4% faster 128-head decode
// than six, the prefill unchanged)
constexpr int kScoreRows = 8;
static_assert(kScoreRows >= 0 && kScoreRows <= kTileSlice, "split of the slice copies");

// Wave index as a scalar: roles branch on it without divergence.
__device__ __forceinline__ uint32_t wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Scorer side.  last(t, nrows) is the last visible tile row of the wave's
// group in tile t (nrows rows of the tile exist).  Scorer s also copies the
// first kScoreRows c_KV rows of slice s of tile t+2 during iteration t (the
// accumulator of that slice copies the rest, its k_r and row maps), from the
// row-map records the accumulator published one barrier earlier, and waits
// for them before the barrier that ends iteration t+1.
template <bool kFlat, class Last>
__device__ __forceinline__ void score_stream(const StreamArgs& ra, SplitSmem& sm, uint32_t g_begin, uint32_t n,
                                             float c, Last&& last, const bf16x8_t (&qb)[18], float& m, float& l) {
  const uint32_t lane = threadIdx.x & 63, s = wave_id(), hq = lane >> 4, hr = lane & 15;
  const uint32_t nt = (n + kTileRows - 1) / kTileRows;
  if (nt == 0) return;
  const WaveSlots<kTileRm, kTileSlice>& ws = sm.s.slots[s];
  const uint32_t row0 = kTileSlice * s;
  __syncthreads();  // tile 0 is in place
  const uint32_t ln = opaque(lane), q = ln >> 4, rr = ln & 15;
  for (uint32_t t = 0; t < nt; ++t) {
    uint32_t src[kScoreRows > 0 ? kScoreRows : 1];
    unsigned char* nx = sm.s.stage[(t + 2) % kStages];
#pragma unroll
    for (int k = 0; k < kScoreRows; ++k) {
      if constexpr (kFlat)
        src[k] = min(g_begin + min(t + 2, nt - 1) * kTileRows + row0 + k, ra.pool_last);
      else
        src[k] = min(ws.rm[(t + 2) % kTileRm][k].x, ra.pool_last);
    }
    const unsigned char* sa = sm.s.stage[t % kStages];
    const unsigned char* rowp = sa + rr * kCkvBytes + ((q ^ (rr & 3)) << 4);
    const unsigned char* base[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) base[i] = rowp + (((uint32_t)i ^ (rr >> 2)) << 6);
    const unsigned char* krp[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) krp[i] = sa + kTileKr + kr_pos(rr, 4 * i + q);
    auto read = [&](int kk, bf16x8_t (&x)[2]) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const unsigned char* ptr = kk < 16 ? base[kk & 3] + 256 * (kk >> 2) + 16 * j * kCkvBytes
                                           : krp[kk - 16] + 16 * j * kKrBytes;
        x[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(ptr));
      }
    };
    // K fragments read ahead of their MFMAs: a shallow ring keeps the LDS queue
    // short for the accumulating waves (2 to 3 measured 5% faster than 8)
    constexpr int kAhead = 2;
    bf16x8_t ring[kAhead + 1][2];
#pragma unroll
    for (int kk = 0; kk < kAhead; ++kk) read(kk, ring[kk]);
    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) {
      if (kk + kAhead < 18) read(kk + kAhead, ring[(kk + kAhead) % (kAhead + 1)]);
      if (kk >= 2 && kk - 2 < kScoreRows) {
        const uint32_t k = kk - 2, r = row0 + k;
        dma16s(pool_row(ra, src[k]), (lane ^ (r & 15)) << 4, lds_addr(nx + r * kCkvBytes));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[kk % (kAhead + 1)][j], qb[kk], acc[j], 0, 0, 0);
    }
    const int32_t lv = last(t, min((uint32_t)kTileRows, n - t * kTileRows));
    float sc[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[j][i] = acc[j][i];
    // lv is the same for the whole wave: only the tiles that reach past the
    // wave's last visible row (the end of a range, a query's own position)
    // need the mask
    if (lv < kTileRows - 1) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((int32_t)(16 * j + 4 * hq + i) > lv) sc[j][i] = -INFINITY;
    }
    float p[2][4], alpha;
    const bool moved = softmax_scores(sc, c, m, l, p, alpha);
    sm.pfrag[t & 1][s][lane] = __builtin_bit_cast(uint4, pack_p8(p[0], p[1]));
    if (hq == 0) sm.alpha[t & 1][s][hr] = alpha;
    if (lane == 0) sm.scaled[t & 1][s] = moved ? 1u : 0u;
    wait_dma_but<kScoreRows>();  // this wave's rows of tile t+1 have landed
    __syncthreads();
  }
  __syncthreads();  // the accumulators' last PV
  wait_dma_all();
}

// Accumulator side: rows [g_begin, g_begin + n) of the assembled sequence.
// sm.s.omega must be visible.  The row-map data an iteration needs (copy
// sources of tile t+2, deltas of tile t+1) is read into registers one
// iteration ahead, so that the only LDS round trip on the way from one
// barrier to the next is the one for the P / C^T fragments and the k_r to
// rotate.
template <bool kFlat>
__device__ __forceinline__ void value_stream(const StreamArgs& ra, SplitSmem& sm, uint32_t g_begin, uint32_t n,
                                             f32x4_t (&o)[kSplitGroups][kSplitNb]) {
  const uint32_t lane = threadIdx.x & 63, j = wave_id() - kSplitGroups, hr = lane & 15;
  const uint32_t nt = (n + kTileRows - 1) / kTileRows;
  if (nt == 0) return;
  WaveSlots<kTileRm, kTileSlice>& ws = sm.s.slots[j];
  const uint32_t row0 = kTileSlice * j;
  int32_t cd[2] = {0, 0};
  auto g0 = [&](uint32_t x) { return g_begin + min(x, nt - 1) * kTileRows + row0; };
  auto stage = [&](uint32_t x) { return sm.s.stage[x % kStages]; };
  auto delta = [&](uint32_t x) -> int32_t {
    if constexpr (kFlat)
      return 0;
    else
      return slice_row_delta<kTileSlice>(ws.rm[x % kTileRm]);
  };
  // copy sources of tile x: from its row map, or consecutive rows (flat)
  auto copies_of = [&](uint32_t x) -> SliceCopies {
    if constexpr (kFlat) {
      SliceCopies c;
      const uint32_t r = g0(x);
#pragma unroll
      for (int k = 0; k < kTileSlice; ++k) c.src[k] = min(r + k, ra.pool_last);
      c.ksrc = min(r + (opaque(lane) >> 3), ra.pool_last);
      return c;
    } else {
      return prep_copies(ra, ws.rm[x % kTileRm]);
    }
  };
  constexpr int kRowMaps = kFlat ? 0 : 1;  // row-map copies per iteration

  SliceCopies cp;  // copy sources of tile t+2
  int32_t d1;      // delta of this lane's row of tile t+1
  // (cos, sin) of the four pairs this lane turns, for delta td: deltas change
  // only at entry boundaries, so most tiles reuse them without an LDS read
  f32x4_t ta = f32x4_t{1.f, 0.f, 1.f, 0.f}, tb = ta;
  int32_t td = 0;

  // Iteration t: wait for tile t+1 and read the P / C^T fragments and the
  // k_r of tile t+1 in one go.  The first half of the PV MFMAs of tile t-1
  // carries the copies of tile t+2; then the rotated k_r is written back and
  // the row-map data of the next iteration read, while the second half runs.
  // The row map of tile t+4 goes out last.  kB: tile t-1 exists (t >= 1).
  auto iteration = [&](uint32_t t, auto kB) {
    constexpr bool B = decltype(kB)::value;
    unsigned char* nx = stage(t + 2);
    unsigned char* sr = stage(t + 1) + kTileKr;
    // Tile t+1 needs turning unless every row of the slice has delta 0
    // (exact-prefix and fresh rows, or a slice past the end).  The trig
    // table holds the rows of the slice's first and last rotated entries
    // (cd), copied one iteration earlier; a slice with a third delta (entries
    // shorter than 8 rows) is turned by slice_rotate, which evaluates the
    // missing deltas in double.
    const bool rot = t + 1 < nt && __any(d1 != 0);
    const bool table = rot && !__any(d1 != 0 && d1 != cd[0] && d1 != cd[1]);
    // Tile t+1 and its trig rows have landed: after them only the row map of
    // tile t+3 went out (t >= 1); at t = 0 nothing did.
    wait_dma_but<B ? kRowMaps : 0>();
    if (rot && !table) slice_rotate<kTileSlice>(ws, sr, row0, sm.s.omega, d1, cd);
    SliceRot rt;
    if (table) {
      if (__any(d1 != td)) {
        const SliceRot x = slice_rot_load(ws, sr, row0, d1, cd);
        ta = x.a;
        tb = x.b;
        td = d1;
        rt.k = x.k;
      } else {
        const uint32_t l = threadIdx.x & 63;
        rt.k = *reinterpret_cast<const u32x4_t*>(sr + kr_pos(row0 + (l >> 3), l & 7));
      }
      rt.a = ta;
      rt.b = tb;
    }
    copy_kr(ra, cp, nx + kTileKr, row0);
    auto mid = [&]() {
      // the table's reads are done once the rotated values are stored
      if (table) slice_rot_store(sr, row0, rt);
      // This iteration's copies of tile t+2 are out; the row map of tile
      // t+3, issued before them, has landed.
      if constexpr (!kFlat) wait_dma_but<kTileSlice - kScoreRows + 1>();
      cp = copies_of(t + 3);
      d1 = delta(t + 2);
      if constexpr (!kFlat) slice_trig_fetch(ra, ws, d1, ws.rm[(t + 2) % kTileRm], cd);
    };
    if constexpr (B) {
      const uint32_t pb = (t - 1) & 1;
      const uint4 scaled = *reinterpret_cast<const uint4*>(sm.scaled[pb]);
      bf16x8_t pf[kSplitGroups];
#pragma unroll
      for (int g = 0; g < kSplitGroups; ++g) pf[g] = __builtin_bit_cast(bf16x8_t, sm.pfrag[pb][g][lane]);
      typedef short i16x8_t __attribute__((ext_vector_type(8)));
      const CtBases c0 = ct_bases(stage(t - 1), 0);
      auto read_cf = [&](int nb) {
        const int nn = kSplitNb * j + nb;
        const i16x4_t lo = ct_read(c0, nn);
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_ptr)(c0.b[nn & 7] + 256 * (nn >> 3) + 16 * kCkvBytes));
        return __builtin_bit_cast(bf16x8_t, (i16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}));
      };
      constexpr int kCfAhead = 3;  // C^T fragments in registers at a time
      bf16x8_t cf[kCfAhead];
#pragma unroll
      for (int nb = 0; nb < kCfAhead; ++nb) cf[nb] = read_cf(nb);
      if (scaled.x | scaled.y | scaled.z | scaled.w) {
#pragma unroll
        for (int g = 0; g < kSplitGroups; ++g) {
          const float a = sm.alpha[pb][g][hr];
#pragma unroll
          for (int nb = 0; nb < kSplitNb; ++nb) o[g][nb] *= a;
        }
      }
#pragma unroll
      for (int nb = 0; nb < kSplitNb; ++nb) {
        // the copies ride on the first half of the column blocks
#pragma unroll
        for (int k = kScoreRows; k < kTileSlice; ++k)
          if ((k - kScoreRows) * (kSplitNb / 2) / (kTileSlice - kScoreRows > 0 ? kTileSlice - kScoreRows : 1) == nb)
            copy_ckv(ra, cp, k, nx, row0);
        const bf16x8_t c = cf[nb % kCfAhead];
        if (nb + kCfAhead < kSplitNb) cf[nb % kCfAhead] = read_cf(nb + kCfAhead);
#pragma unroll
        for (int g = 0; g < kSplitGroups; ++g)
          o[g][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c, pf[g], o[g][nb], 0, 0, 0);
        if (nb == kSplitNb / 2 - 1) mid();
      }
    } else {
#pragma unroll
      for (int k = kScoreRows; k < kTileSlice; ++k) copy_ckv(ra, cp, k, nx, row0);
      mid();
    }
    if constexpr (!kFlat) slice_issue_rowmap<kTileSlice>(ra, g0(t + 4), ws.rm[(t + 4) % kTileRm]);
    __syncthreads();
  };

  if constexpr (!kFlat) {
    for (uint32_t x = 0; x < 4; ++x) slice_issue_rowmap<kTileSlice>(ra, g0(x), ws.rm[x]);
    wait_dma_all();
  }
  for (uint32_t x = 0; x < 2; ++x) {  // copies of tiles 0 and 1 (iterations 0, 1 fetch row maps 4, 5)
    const SliceCopies c = copies_of(x);
#pragma unroll
    for (int k = 0; k < kTileSlice; ++k) copy_ckv(ra, c, k, stage(x), row0);
    copy_kr(ra, c, stage(x) + kTileKr, row0);
  }
  cp = copies_of(2);
  d1 = delta(1);
  wait_dma_but<kTileSlice + 1>();  // tile 0 has landed (tile 1's copies may be outstanding)
  slice_rotate<kTileSlice>(ws, stage(0) + kTileKr, row0, sm.s.omega, delta(0), cd);
  if constexpr (!kFlat) slice_trig_fetch(ra, ws, d1, ws.rm[1], cd);  // trig rows of tile 1
  __syncthreads();
  iteration(0, std::false_type{});
  for (uint32_t t = 1; t <= nt; ++t) iteration(t, std::true_type{});
  wait_dma_all();
}

}  // namespace dev
}  // namespace irm
