// Non-absorbed MLA prefill, attention: every head attends with its own
// 192-wide key [k_nope | k_r] and 128-wide value, both up-projected from the
// latent rows beforehand (irm_upproj.hip) (Irminsul pages: gentlecold.top
// article, section 4 for the key [W_UK c_KV, k_r] and the value from c_KV;
// section 13 for the non-absorbed form, which has to up-project c_KV at run
// time).  k_r is the rotated slice of the assembled row, shared by all heads;
// only it carries the position.
//
// mha_prefill_kernel: causal attention of 256 queries of one head per
// workgroup of eight waves over the head's rows, streamed in 64-row tiles
// through two LDS stages with one barrier per tile (one workgroup per compute
// unit: each tile copied into LDS serves eight waves, measured 8% faster than
// two four-wave workgroups of 128 queries; 64-row tiles measured 12% faster
// than 32-row tiles in three or four stages).

#include <hip/hip_runtime.h>

#include "irm_attn.h"
#include "irm_launch.h"

namespace irm {
namespace {

using namespace irm::dev;

// LDS offset of 16-byte unit u of row r in a tile of 128-byte rows: units
// are permuted by (r >> 1) & 7, so 16 lanes reading one unit of 16
// consecutive rows cover all 64 banks.
__device__ __forceinline__ uint32_t pos128(uint32_t r, uint32_t u) { return r * 128 + ((u ^ ((r >> 1) & 7)) << 4); }

// ---------------------------------------------------------------------------
// per-head causal prefill
//
// Workgroup = (head h, 32 W queries); wave w owns queries 32w .. 32w+31 as two
// 16-query blocks and walks every tile of the keys they can see.  Scores are
// S^T = K Q^T (lane (q, r): keys 4q..4q+3 of a 16-key block for query r), so
// each lane holds 4 scores per key block and query block, and the maximum
// over a query's keys is a maximum over the four lane quarters.  O^T = V^T P^T
// leaves every lane with value dims 4q..4q+3 of one query, so the rescale is
// lane-local.  P of two key blocks feeds one 32-deep MFMA in the lane's k
// order {4q..4q+3, 16+4q..16+4q+3}.
//
// Stage of T keys: k_nope [T][256 B] (unit c of row r at c ^ (r & 15)),
// k_r [T][128 B] (pos128), v [T][256 B] (unit c of row r at c ^ (2r & 15):
// the transposing reads of 8 consecutive rows then cover all 64 banks, where
// k_nope's swizzle left them 2-way conflicted).  Wave w copies rows
// wT/W .. (w+1)T/W - 1 of each part with 1 KB LDS-DMA copies.  With S
// stages, tiles t+1 .. t+S-1 are in flight while tile t is computed, and one
// barrier per tile both publishes tile t and frees the stage of tile t-1.
// ---------------------------------------------------------------------------
template <int T, int W>
struct MhaTile {
  static constexpr int kKn = T * 256;
  static constexpr int kKr = T * 128;
  static constexpr int kBytes = 2 * kKn + kKr;
  static constexpr int kRows = T / W;                          // rows per wave
  static constexpr int kCopies = 2 * (kRows / 4) + kRows / 8;  // 1 KB copies per wave
  static constexpr int kBlocks = T / 16;                       // 16-key blocks
  static constexpr int kQ = 32 * W;                            // queries per workgroup
  static_assert(kRows % 8 == 0, "whole k_r copies per wave");
};

struct MhaArgs {
  const unsigned char* q_nope;  // bf16 [n_q][H][128]
  const unsigned char* q_rope;  // bf16 [n_q][H][64]
  const unsigned char* kv;      // bf16 [rows][576] (k_r at byte 1024)
  const unsigned char* kvh;     // bf16 [H][rows][256] = [k_nope | v]
  unsigned char* out;           // bf16 [n_q][H][128]
  float* lse;                   // [n_q][H] or null
  uint32_t rows, n_heads, n_q, q_blocks;
  int32_t q_pos0;
  float c;                      // scale * log2(e)
};

template <int T, int W>
__device__ __forceinline__ void mha_issue(const MhaArgs& a, unsigned char* st, uint32_t h, uint32_t t0) {
  using Tl = MhaTile<T, W>;
  const uint32_t lane = opaque(threadIdx.x & 63), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // row bases of the tile in scalar registers, 32-bit lane offsets (rows past
  // the last are clamped to it)
  const unsigned char* hb = a.kvh + ((size_t)h * a.rows + t0) * 512;
  const unsigned char* kb = a.kv + (size_t)t0 * kRowBytes + kCkvBytes;
  const uint32_t last = a.rows - 1 - t0;
  const uint32_t rw = w * Tl::kRows;
#pragma unroll
  for (int i = 0; i < Tl::kRows / 4; ++i) {
    const uint32_t r = rw + 4 * i + (lane >> 4);
    const uint32_t rb = min(r, last) * 512;
    dma16s(hb, rb + 16 * ((lane & 15) ^ (r & 15)), lds_addr(st + (rw + 4 * i) * 256));  // k_nope
    dma16s(hb + 256, rb + 16 * ((lane & 15) ^ (2 * r & 15)),
           lds_addr(st + Tl::kKn + Tl::kKr + (rw + 4 * i) * 256));                      // v
  }
#pragma unroll
  for (int i = 0; i < Tl::kRows / 8; ++i) {
    const uint32_t r = rw + 8 * i + (lane >> 3);
    dma16s(kb, min(r, last) * kRowBytes + 16 * ((lane & 7) ^ ((r >> 1) & 7)), lds_addr(st + Tl::kKn + (rw + 8 * i) * 128));
  }
}

// Online softmax of one query block over NB key blocks (the branch-free form
// of softmax_scores in irm_attn.h): leaves p and alpha, returns whether any
// query's reference maximum moved.
template <int NB>
__device__ __forceinline__ bool softmax_blocks(const float (&s)[NB][4], float c, float& m, float& l,
                                               float (&p)[NB][4], float& alpha) {
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < NB; ++j)
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
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[j][i] = __builtin_amdgcn_exp2f(fmaf(s[j][i], c, -m_use));
      sum += p[j][i];
    }
  l += sum;
  return __any(mv);
}

// Per-lane LDS offsets within a stage, from a lane id the compiler must
// treat as fresh (so they are formed where used, not held across the loop):
// the K reads of score step kk (0-3 k_nope unit (4kk + q) ^ rr of row rr,
// 4-5 k_r) and the transposing V reads of value block vb (as ct_bases in
// irm_attn.h, here on 256-byte rows: lane (q, s) reads row x = 4q + s/4, 8
// bytes of unit 2vb + hh, hh = (s % 4) / 2, which sits at position
// (2vb + hh) ^ (2x & 15) = 2 (vb ^ (x & 7)) + hh).  Key block j adds an
// immediate.
template <int T, int W>
__device__ __forceinline__ void mha_k_offsets(uint32_t (&k)[6]) {
  using Tl = MhaTile<T, W>;
  const uint32_t lane = opaque(threadIdx.x & 63), q = lane >> 4, rr = lane & 15;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) k[kk] = rr * 256 + ((((uint32_t)(4 * kk) + q) ^ rr) << 4);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) k[4 + kk] = Tl::kKn + pos128(rr, 4 * kk + q);
}

template <int T, int W>
__device__ __forceinline__ void mha_v_offsets(uint32_t (&v)[8]) {
  using Tl = MhaTile<T, W>;
  const uint32_t lane = opaque(threadIdx.x & 63), q = lane >> 4, rr = lane & 15;
  const uint32_t x = 4 * q + (rr >> 2), hh = (rr & 3) >> 1;
  const uint32_t rowo = Tl::kKn + Tl::kKr + x * 256 + (hh << 4) + 8 * (rr & 1);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = rowo + (((uint32_t)i ^ (x & 7)) << 5);
}

// One tile: scores, online softmax (kMask: some key of the tile lies past
// some query of the wave), value products.
template <int T, int W, bool kMask>
__device__ __forceinline__ void mha_tile(const unsigned char* st, const bf16x8_t (&qf)[2][6],
                                         f32x4_t (&o)[8][2], float (&m)[2], float (&l)[2], uint32_t t0,
                                         int32_t lim0, float c) {
  using Tl = MhaTile<T, W>;
  constexpr int NB = Tl::kBlocks;
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const uint32_t q = (threadIdx.x & 63) >> 4;
  uint32_t koff[6];
  mha_k_offsets<T, W>(koff);

  // scores: S^T of key blocks j for query blocks b
  f32x4_t s[2][NB];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int j = 0; j < NB; ++j) s[b][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 6; ++kk) {
    const unsigned char* p = st + koff[kk];
    bf16x8_t kf[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      kf[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p + (kk < 4 ? 16 * j * 256 : 16 * j * 128)));
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < NB; ++j) s[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[j], qf[b][kk], s[b][j], 0, 0, 0);
  }

  // online softmax per query block
  bf16x8_t pb[2][NB / 2];
  // key t0 + 16j + 4q + i is past query qw + 16b + r when 16j + i > d + 16b
  const int32_t d = kMask ? (int32_t)opaque((uint32_t)(lim0 - (int32_t)(t0 + 4 * q))) : 0;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float sv[NB][4], p[NB][4], alpha;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (kMask) {
          sv[j][i] = 16 * j + i > d + 16 * b ? -INFINITY : s[b][j][i];
        } else {
          sv[j][i] = s[b][j][i];
        }
      }
    if (softmax_blocks<NB>(sv, c, m[b], l[b], p, alpha)) {
#pragma unroll
      for (int vb = 0; vb < 8; ++vb) o[vb][b] *= alpha;
    }
#pragma unroll
    for (int pi = 0; pi < NB / 2; ++pi) pb[b][pi] = pack_p8(p[2 * pi], p[2 * pi + 1]);
  }

  // O^T += V^T P^T, one 32-deep MFMA per pair of key blocks
  uint32_t voff[8];
  mha_v_offsets<T, W>(voff);
#pragma unroll
  for (int pi = 0; pi < NB / 2; ++pi)
#pragma unroll
    for (int vb = 0; vb < 8; ++vb) {
      const unsigned char* base = st + voff[vb] + pi * 32 * 256;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)base);
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(base + 16 * 256));
      const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, i16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
      for (int b = 0; b < 2; ++b) o[vb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[b][pi], o[vb][b], 0, 0, 0);
    }
}

template <int T, int S, int W>
__global__ __launch_bounds__(64 * W, 8 / W) void mha_prefill_kernel(MhaArgs a) {
  using Tl = MhaTile<T, W>;
  constexpr uint32_t kMhaQ = Tl::kQ;
  __shared__ unsigned char smem[S][Tl::kBytes];
  const uint32_t h = blockIdx.x % a.n_heads;
  const uint32_t qblk = a.q_blocks - 1 - blockIdx.x / a.n_heads;  // longest blocks first
  const uint32_t lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t q = lane >> 4, r = lane & 15;
  const uint32_t qw = qblk * kMhaQ + 32 * w;                     // first query of the wave
  const uint32_t q_last = min(qblk * kMhaQ + kMhaQ, a.n_q) - 1;  // last valid query of the workgroup
  const uint32_t n_keys = (uint32_t)a.q_pos0 + q_last + 1;
  const uint32_t n_tiles = (n_keys + T - 1) / T;

  // Q^T operands: block b, step kk (0-3 nope, 4-5 rope), lane (q, r) holds
  // dims 32kk + 8q .. +8 of query qw + 16b + r (clamped past the last query)
  bf16x8_t qf[2][6];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint32_t qi = min(qw + 16 * b + r, a.n_q - 1);
    const uint4* pn = reinterpret_cast<const uint4*>(a.q_nope + ((size_t)qi * a.n_heads + h) * 256) + q;
    const uint4* pr = reinterpret_cast<const uint4*>(a.q_rope + ((size_t)qi * a.n_heads + h) * 128) + q;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[b][kk] = __builtin_bit_cast(bf16x8_t, pn[4 * kk]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) qf[b][4 + kk] = __builtin_bit_cast(bf16x8_t, pr[4 * kk]);
  }
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int kk = 0; kk < 6; ++kk) asm volatile("" : "+v"(qf[b][kk]));

  f32x4_t o[8][2];
#pragma unroll
  for (int vb = 0; vb < 8; ++vb)
#pragma unroll
    for (int b = 0; b < 2; ++b) o[vb][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  // a query at position q_pos0 + i sees keys t <= q_pos0 + i
  const int32_t lim0 = a.q_pos0 + (int32_t)(qw + r);
  const uint32_t first_masked = (uint32_t)a.q_pos0 + qw + 1;  // tiles ending at or below this need no mask

#pragma unroll
  for (int i = 0; i < S - 1; ++i)
    if ((uint32_t)i < n_tiles) mha_issue<T, W>(a, smem[i], h, i * T);
  for (uint32_t t = 0; t < n_tiles; ++t) {
    // copies of tiles t+1 .. t+S-2 may stay in flight
    const uint32_t ahead = min(n_tiles - 1 - t, (uint32_t)(S - 2));
    if (S >= 4 && ahead >= 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * Tl::kCopies) : "memory");
    else if (S >= 3 && ahead >= 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Tl::kCopies) : "memory");
    else
      wait_dma_all();
    __syncthreads();  // tile t is in LDS; every wave is done with tile t - 1
    if (t + S - 1 < n_tiles) mha_issue<T, W>(a, smem[(t + S - 1) % S], h, (t + S - 1) * T);
    const uint32_t t0 = t * T;
    if (t0 + T > first_masked)
      mha_tile<T, W, true>(smem[t % S], qf, o, m, l, t0, lim0, a.c);
    else
      mha_tile<T, W, false>(smem[t % S], qf, o, m, l, t0, lim0, a.c);
  }

  // normalise and store: lane (q, r) holds value dims 16vb + 4q .. +3 of query qw + 16b + r
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float lt = l[b];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const uint32_t qi = qw + 16 * b + r;
    if (qi >= a.n_q) continue;
    const float inv = 1.f / lt;
    unsigned char* dst = a.out + ((size_t)qi * a.n_heads + h) * 256 + 8 * q;
#pragma unroll
    for (int vb = 0; vb < 8; ++vb) {
      const f32x4_t& x = o[vb][b];
      *reinterpret_cast<uint2*>(dst + 32 * vb) =
          make_uint2(pack_bf16(x[0] * inv, x[1] * inv), pack_bf16(x[2] * inv, x[3] * inv));
    }
    if (a.lse && q == 0) a.lse[(size_t)qi * a.n_heads + h] = (m[b] + __log2f(lt)) * kLn2;
  }
}

// tile shape of the launch: keys per tile, LDS stages
constexpr int kMhaT = 64;
constexpr int kMhaS = 2;
constexpr int kMhaW = 8;
using MhaLaunch = MhaTile<kMhaT, kMhaW>;
static_assert(kMhaS * MhaLaunch::kBytes * (8 / kMhaW) <= 160 * 1024, "the workgroups of a compute unit fit the LDS");
static_assert(kMhaS >= 2 && kMhaS <= 4, "stage count");

}  // namespace

irm_status launch_prefill_nonabsorbed(const void* q_nope, const void* q_rope, int32_t q_pos0, uint32_t n_q,
                                      const void* kv, const void* kvh, uint64_t kv_rows, uint32_t n_heads,
                                      float scale, void* out, float* lse, hipStream_t s) {
  MhaArgs a;
  a.q_nope = static_cast<const unsigned char*>(q_nope);
  a.q_rope = static_cast<const unsigned char*>(q_rope);
  a.kv = static_cast<const unsigned char*>(kv);
  a.kvh = static_cast<const unsigned char*>(kvh);
  a.out = static_cast<unsigned char*>(out);
  a.lse = lse;
  a.rows = (uint32_t)kv_rows;
  a.n_heads = n_heads;
  a.n_q = n_q;
  a.q_blocks = (n_q + MhaLaunch::kQ - 1) / MhaLaunch::kQ;
  a.q_pos0 = q_pos0;
  a.c = scale * kLog2e;
  hipLaunchKernelGGL((mha_prefill_kernel<kMhaT, kMhaS, kMhaW>), dim3(a.q_blocks * n_heads), dim3(64 * kMhaW), 0, s, a);
  return launch_check("non-absorbed prefill kernel");
}

}  // namespace irm
