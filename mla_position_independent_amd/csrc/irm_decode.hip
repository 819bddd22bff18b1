// Split-KV MLA decode with the delta rotation applied while KV rows are
// loaded, and the pass that combines the splits.
//
// Irminsul pages: the rotation k_r = R(p_tgt - p_src) k_r_base of registry
// hits (gist.science summary, sections 2.1 and 2.2), fused into the load of
// the KV tile as the pages propose for the HBM-to-on-chip path (gist.science,
// sections 2.2 and 4; gentlecold.top article, sections 5 and 14.1); absorbed
// MLA attention per query token (gentlecold.top, section 4).

#include <hip/hip_runtime.h>

#include "irm_attn.h"
#include "irm_launch.h"

namespace irm {
namespace {

using namespace irm::dev;

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

StreamArgs stream_args(const irm_table* t, const void* pool, uint64_t pool_rows) {
  StreamArgs ra;
  ra.pool = static_cast<const unsigned char*>(pool);
  ra.rowmap = image_of(t).rowmap;
  ra.pool_last = pool_last_of(pool_rows);
  return ra;
}

}  // namespace

uint32_t decode_default_splits(const irm_table* t, uint32_t n_groups) {
  // one workgroup per CU (256 CUs) with >= 256 rows per split
  const uint32_t want = (256 + t->n_seq * n_groups - 1) / (t->n_seq * n_groups);
  const uint32_t cap = (t->max_seq_len + 255) / 256;
  uint32_t s = want < cap ? want : cap;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return s;
}

irm_status launch_decode(const irm_table* t, const void* q_lat, const void* q_rope, const void* pool,
                         uint64_t pool_rows, uint32_t n_heads, uint32_t n_splits, float scale, void* out,
                         float* lse, float* ws_acc, float* ws_ml, hipStream_t s) {
  const uint32_t G = n_heads / 16;
  DecodeArgs a;
  a.ra = stream_args(t, pool, pool_rows);
  a.seq_base = image_of(t).seq_base;
  a.q_lat = static_cast<const uint4*>(q_lat);
  a.q_rope = static_cast<const uint4*>(q_rope);
  a.ws_acc = ws_acc;
  a.ws_ml = ws_ml;
  a.n_seq = t->n_seq;
  a.n_heads = n_heads;
  a.n_groups = G;
  a.n_splits = n_splits;
  a.scale_log2 = scale * kLog2e;
  for (int i = 0; i < (int)kPairs; ++i) a.f.w[i] = t->inv_freq[i];
  const uint64_t bs = (uint64_t)t->n_seq * n_splits;
  const uint64_t grid = (bs + 7) / 8 * 8 * G;
  if (grid > 0x7fffffffull) return fail(IRM_EUNSUPPORTED, "irm_mla_decode: grid too large");
  hipLaunchKernelGGL(decode_split_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, s, a);
  irm_status st = launch_check("irm_mla_decode: split kernel");
  if (st != IRM_OK) return st;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(t->n_seq * n_heads), dim3(128), 0, s, ws_acc, ws_ml,
                     static_cast<uint16_t*>(out), lse, n_heads, n_splits);
  return launch_check("irm_mla_decode: combine kernel");
}

}  // namespace irm
