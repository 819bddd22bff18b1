// Device-side definitions shared by the HIP sources: sizes, vector types,
// the device image of a chunk table, bf16 helpers and the 2x2 rotation.
//
// Data layout: pool and assembled rows are bf16 [rows][576] = 72 units of
// 16 bytes; units 0..63 are c_KV, units 64..71 are k_r (4 rotation pairs per
// unit).  Angles are formed and their sine/cosine evaluated in double (delta
// reaches 2^17, where a float angle is off by ~1e-2 rad); only the 2x2
// rotation itself runs in float.
#pragma once

#include <hip/hip_runtime.h>

#include "irm_internal.h"

namespace irm {
namespace dev {

constexpr int kRowBytes = IRM_ROW * 2;                       // 1152
constexpr int kUnitsPerRow = kRowBytes / 16;                 // 72
constexpr int kLatUnits = IRM_D_LATENT * 2 / 16;             // 64
constexpr int kThreads = 256;                                // 4 waves of 64
constexpr int kTile = 64;                                    // KV rows per tile
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
  const GatherGroup* groups;
  const uint32_t* members;
  const uint4* items;   // {first pool row, rows | members << 4, first member, row offset}
  uint32_t n_entries;
};


inline Image image_of(const irm_table* t) {
  const unsigned char* d = static_cast<const unsigned char*>(t->dev);
  Image im;
  im.ents = reinterpret_cast<const DevEntry*>(d + t->layout.off_entries);
  im.seq_first = reinterpret_cast<const uint32_t*>(d + t->layout.off_seq_first);
  im.seq_base = reinterpret_cast<const uint32_t*>(d + t->layout.off_seq_base);
  im.block_map = reinterpret_cast<const uint32_t*>(d + t->layout.off_block_map);
  im.trig = reinterpret_cast<const float2*>(d + t->layout.off_trig);
  im.rowmap = reinterpret_cast<const uint4*>(d + t->layout.off_rowmap);
  im.groups = reinterpret_cast<const GatherGroup*>(d + t->layout.off_groups);
  im.members = reinterpret_cast<const uint32_t*>(d + t->layout.off_members);
  im.items = reinterpret_cast<const uint4*>(d + t->layout.off_items);
  im.n_entries = t->n_chunks;
  return im;
}

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 (lo in bits 0-15), round to nearest even, in
// one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
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


}  // namespace dev
}  // namespace irm
