// Device building blocks shared by the attention kernels: HBM -> LDS copies
// and the MFMA score / value products with the online softmax.
//
// Absorbed MLA attention (Irminsul pages: gentlecold.top article, section 4):
// score = q_lat . c_KV + q_rope . k_r over the 576-wide row, value = c_KV.
#pragma once

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

}  // namespace dev
}  // namespace irm
