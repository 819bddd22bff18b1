// Split-KV MLA decode with the delta rotation applied while KV rows are
// loaded, and the pass that combines the splits.
//
// Irminsul pages: the rotation k_r = R(p_tgt - p_src) k_r_base of registry
// hits (gist.science summary, sections 2.1 and 2.2), fused into the load of
// the KV tile as the pages propose for the HBM-to-on-chip path (gist.science,
// sections 2.2 and 4; gentlecold.top article, sections 5 and 14.1); absorbed
// MLA attention per query token (gentlecold.top, section 4).

#include <hip/hip_runtime.h>

#include <mutex>

#include "irm_attn.h"
#include "irm_launch.h"

// Partial states of the split pass for callers that cannot allocate: one
// array per device, held until the process ends.  Host code never passes
// `scratch` itself to a kernel (on the host it only names the symbol); it
// passes the device address decode_scratch() looks up once per device.
static __device__ __align__(256) unsigned char scratch[irm::kDecodeScratchBytes];

namespace irm {
namespace {

using namespace irm::dev;

struct DecodeArgs {
  StreamArgs ra;
  const uint32_t* seq_base;
  const uint4* q_lat;
  const uint4* q_rope;
  float* ws_acc;  // [n_seq][n_parts][n_heads][512], unnormalised
  float* ws_ml;   // [n_seq][n_parts][n_heads][2]: base-2 max, sum
  uint32_t n_seq, n_heads, n_groups, n_splits;
  uint32_t splits_per_wg;  // shared-tile kernel: consecutive splits per workgroup (divides n_splits);
                           // n_parts = n_splits / splits_per_wg partial states per sequence
  float scale_log2;
  InvFreq f;
};

// Rows [r0, r1) of the split sp of a sequence with N rows: splits are whole
// multiples of 64 rows so that every wave range and tile is aligned.
__device__ __forceinline__ uint32_t split_len(uint32_t N, uint32_t n_splits) {
  return ((N + n_splits - 1) / n_splits + 63) / 64 * 64;
}

__device__ __forceinline__ void split_rows(uint32_t N, uint32_t n_splits, uint32_t sp, uint32_t& r0, uint32_t& r1) {
  const uint32_t per = split_len(N, n_splits);
  r0 = min(N, sp * per);
  r1 = min(N, r0 + per);
}

// Raw scores of one 16-row block for 16 heads, -inf from row nvalid on.
__device__ __forceinline__ void mask_rows(const f32x4_t& acc, uint32_t row0, uint32_t nvalid, float (&sc)[4]) {
  const uint32_t hq = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] = (row0 + 4 * hq + i < nvalid) ? acc[i] : -INFINITY;
}

// ---------------------------------------------------------------------------
// split-KV decode, pass 1, one 16-head group per workgroup: wave-private
// streams
//
// Workgroup = (sequence, split, 16-head group), 4 waves, one workgroup per
// CU.  The split's rows are cut into four contiguous ranges, one per wave,
// and every wave streams its range on its own in 16-row slices through a
// private two-stage LDS ring, rotates k_r in place, scores the 16 rows for
// its 16 heads and accumulates all 512 output columns.  Nothing in the slice
// loop waits for another wave; the four online-softmax states merge once at
// the end.  Per iteration t a wave issues the row map of slice t+3 and the
// data of slice t+1, then waits until at most those 19 copies are
// outstanding, which means slice t has landed.
// ---------------------------------------------------------------------------
constexpr int kPrivRows = 16;
constexpr int kPrivStageKr = kPrivRows * kCkvBytes;
constexpr int kPrivStageBytes = kPrivRows * (kCkvBytes + kKrBytes);  // 18432

constexpr int kPrivRm = 4;  // row-map slots per wave

struct PrivateSmem {
  unsigned char stage[4][2][kPrivStageBytes];
  WaveSlots<kPrivRm, kPrivRows> slots[4];
  double omega[kPairs];
  float ml[4][16][2];
};

__global__ __launch_bounds__(kThreads, 1) void decode_private_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) PrivateSmem sm;

  // Workgroups of the same (sequence, split) but different head groups get
  // the same x % 8, i.e. the same XCD and L2, at consecutive slots.
  const uint32_t x = blockIdx.x, xcd = x & 7, slot = x >> 3;
  const uint32_t g = slot % a.n_groups;
  const uint32_t bs = (slot / a.n_groups) * 8 + xcd;
  if (bs >= a.n_seq * a.n_splits) return;
  const uint32_t b = bs / a.n_splits, sp = bs % a.n_splits;

  const uint32_t base = a.seq_base[b];
  uint32_t r0, r1;
  split_rows(a.seq_base[b + 1] - base, a.n_splits, sp, r0, r1);

  const int lane = threadIdx.x & 63, wave = (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hq = lane >> 4, hr = lane & 15;
  const uint32_t head = g * 16 + hr;

  // this wave's rows: a quarter of the split, in whole slices
  const uint32_t quarter = ((r1 - r0 + 3) / 4 + kPrivRows - 1) / kPrivRows * kPrivRows;
  const uint32_t w0 = min(r1, r0 + wave * quarter), w1 = min(r1, w0 + quarter);
  const uint32_t g_begin = base + w0, n = w1 - w0;
  const uint32_t nt = (n + kPrivRows - 1) / kPrivRows;
  WaveSlots<kPrivRm, kPrivRows>& ws = sm.slots[wave];
  auto g0 = [&](uint32_t t) { return g_begin + min(t, nt - 1) * kPrivRows; };

  // The row maps of the first slices go out before the query loads, so that
  // both round trips overlap (the loads' waits cover the older copies).
  if (nt > 0)
    for (uint32_t t = 0; t < 3; ++t) slice_issue_rowmap<kPrivRows>(a.ra, g0(t), ws.rm[t]);
  bf16x8_t qb[18];
  load_q(a.q_lat, a.q_rope, b, a.n_heads, head, qb);
  fill_omega(sm.omega, a.f);
  f32x4_t o[32];
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  int32_t cd[2] = {0, 0};  // deltas held in the wave's trig table
  __syncthreads();

  if (nt > 0) {
    wait_dma_all();
    slice_issue_data<kPrivRows>(a.ra, ws.rm[0], sm.stage[wave][0], sm.stage[wave][0] + kPrivStageKr, 0);
    for (uint32_t t = 0; t < nt; ++t) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of the stage about to be refilled are done
      slice_issue_rowmap<kPrivRows>(a.ra, g0(t + 3), ws.rm[(t + 3) % kPrivRm]);
      if (t + 1 < nt) {
        unsigned char* nx = sm.stage[wave][(t + 1) & 1];
        slice_issue_data<kPrivRows>(a.ra, ws.rm[(t + 1) % kPrivRm], nx, nx + kPrivStageKr, 0);
        wait_dma_but<19>();
      } else {
        wait_dma_but<1>();
      }
      unsigned char* st = sm.stage[wave][t & 1];
      slice_rotate<kPrivRows>(ws, st + kPrivStageKr, 0, sm.omega, slice_row_delta<kPrivRows>(ws.rm[t % kPrivRm]), cd);
      f32x4_t acc[1];
      qk_blocks<1>(st, st + kPrivStageKr, 0, qb, acc);
      float sc[1][4] = {{acc[0][0], acc[0][1], acc[0][2], acc[0][3]}};
      const uint32_t nv = n - t * kPrivRows;
      if (nv < (uint32_t)kPrivRows) mask_rows(acc[0], 0, nv, sc[0]);
      float p[1][4];
      softmax_update_n<1, 32>(sc, a.scale_log2, m, l, o, p);
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
  // [4 waves][16 heads][128 quads of 4 floats]; quad u of head h's row sits
  // at u ^ h, so that the 16 heads a wave's lanes write at once fall in 16
  // different bank groups (unswizzled, the 2 KB row stride put them all in
  // one: a 16-way conflict on every write, measured 3.3 us per workgroup)
  float* red = reinterpret_cast<float*>(&sm.stage[0][0][0]);
  static_assert(4 * 16 * IRM_D_LATENT * 4 <= sizeof(sm.stage), "merge buffer fits the rings");
  float* mine = red + wave * 16 * IRM_D_LATENT;
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) {
    float4 v = make_float4(fw * o[nb][0], fw * o[nb][1], fw * o[nb][2], fw * o[nb][3]);
    *reinterpret_cast<float4*>(mine + hr * IRM_D_LATENT + 4 * ((4 * nb + hq) ^ hr)) = v;
  }
  __syncthreads();
  const size_t pidx = ((size_t)b * a.n_splits + sp) * a.n_heads + g * 16;
  float4* dst = reinterpret_cast<float4*>(a.ws_acc + pidx * IRM_D_LATENT);
  const float4* src = reinterpret_cast<const float4*>(red);
  constexpr int kQuads = 16 * IRM_D_LATENT / 4;
  constexpr int kRowQuads = IRM_D_LATENT / 4;
  for (int i = threadIdx.x; i < kQuads; i += kThreads) {
    const int h = i / kRowQuads, j = h * kRowQuads + ((i % kRowQuads) ^ h);
    const float4 v0 = src[j], v1 = src[j + kQuads], v2 = src[j + 2 * kQuads], v3 = src[j + 3 * kQuads];
    dst[i] = make_float4(v0.x + v1.x + v2.x + v3.x, v0.y + v1.y + v2.y + v3.y, v0.z + v1.z + v2.z + v3.z,
                         v0.w + v1.w + v2.w + v3.w);
  }
  if (threadIdx.x < 16) {
    a.ws_ml[(pidx + threadIdx.x) * 2 + 0] = mstar;
    a.ws_ml[(pidx + threadIdx.x) * 2 + 1] = (mstar == -INFINITY) ? 0.f : lsum;
  }
}

// ---------------------------------------------------------------------------
// split-KV decode, pass 1, four 16-head groups per workgroup: shared tiles
//
// Workgroup = (sequence, run of U consecutive splits, 64-head block) of eight
// waves.  Scoring wave s holds head group 4 blk + s; accumulating wave j sums
// columns 128 j .. 128 j + 127 of all four groups (score_stream /
// value_stream), so the KV is copied once per 64 heads instead of once per
// 16.  The U splits are contiguous rows, streamed as one softmax run, which
// keeps the copy pipeline full and pays the workgroup's start-up once; the
// run's partial state goes to the workspace as one part (O from the
// accumulating waves, (m, l) from the scoring waves), so the combine pass
// reads n_splits / U parts per sequence.  A run without rows leaves the
// empty state (O = 0, m = -inf, l = 0).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRoleThreads, 1) void decode_shared_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) SplitSmem sm;

  const uint32_t n_blk = a.n_groups / kSplitGroups;
  const uint32_t U = a.splits_per_wg, n_runs = a.n_splits / U;
  const uint32_t x = blockIdx.x, xcd = x & 7, slot = x >> 3;
  const uint32_t hb = slot % n_blk;
  const uint32_t br = (slot / n_blk) * 8 + xcd;
  if (br >= a.n_seq * n_runs) return;
  const uint32_t b = br / n_runs, run = br % n_runs;

  const uint32_t base = a.seq_base[b], N = a.seq_base[b + 1] - base;
  const uint32_t per = split_len(N, a.n_splits);
  const uint32_t r0 = min(N, run * U * per), r1 = min(N, r0 + U * per);

  const uint32_t lane = threadIdx.x & 63, w = wave_id(), hq = lane >> 4, hr = lane & 15;
  const uint32_t g0 = hb * kSplitGroups;  // first head group of the block
  const size_t pbase = (size_t)br * a.n_heads + g0 * 16;  // part (b, run) of the first head
  fill_omega(sm.s.omega, a.f);

  if (w < kSplitGroups) {  // scoring wave: head group g0 + w
    bf16x8_t qb[18];
    load_q<false>(a.q_lat, a.q_rope, b, a.n_heads, (g0 + w) * 16 + hr, qb);
    float m = -INFINITY, l = 0.f;
    __syncthreads();
    score_stream<false>(a.ra, sm, base + r0, r1 - r0, a.scale_log2,
                        [&](uint32_t, uint32_t nrows) -> int32_t { return (int32_t)nrows - 1; }, qb, m, l);
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (hq == 0) {
      float* d = a.ws_ml + (pbase + 16 * w + hr) * 2;
      d[0] = m;
      d[1] = (m == -INFINITY) ? 0.f : l;
    }
    return;
  }

  // accumulating wave j: partial O of the four groups over columns 128 j ..
  const uint32_t j = w - kSplitGroups;
  f32x4_t o[kSplitGroups][kSplitNb];
#pragma unroll
  for (int g = 0; g < kSplitGroups; ++g)
#pragma unroll
    for (int nb = 0; nb < kSplitNb; ++nb) o[g][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  value_stream<false>(a.ra, sm, base + r0, r1 - r0, o);
#pragma unroll
  for (int g = 0; g < kSplitGroups; ++g) {
    float* dst = a.ws_acc + (pbase + 16 * g + hr) * IRM_D_LATENT + kSplitCols * j + 4 * hq;
#pragma unroll
    for (int nb = 0; nb < kSplitNb; ++nb)
      *reinterpret_cast<float4*>(dst + 16 * nb) = make_float4(o[g][nb][0], o[g][nb][1], o[g][nb][2], o[g][nb][3]);
  }
}

// ---------------------------------------------------------------------------
// split-KV decode, pass 2
// ---------------------------------------------------------------------------
// One workgroup per (sequence, head), one float4 of the 512 columns per
// thread, over the n_parts partial states of the sequence (one per split, or
// one per run of splits of the 64-head kernel).  kMax > 0: at most kMax
// parts, every load issued before any arithmetic; kMax = 0: any count, in
// batches.  Every part holds finite values (zeros for a part without rows,
// whose maximum is -inf and whose weight is 0), so no load depends on
// another part's values.
template <int kMax>
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ ws_acc,
                                                             const float* __restrict__ ws_ml,
                                                             uint16_t* __restrict__ out,
                                                             float* __restrict__ lse,
                                                             uint32_t n_heads, uint32_t n_parts) {
  const uint32_t bh = blockIdx.x;
  const uint32_t b = bh / n_heads, h = bh % n_heads;
  const size_t p0 = (size_t)b * n_parts * n_heads + h;  // part s: p0 + s * n_heads
  const float2* ml = reinterpret_cast<const float2*>(ws_ml);
  auto acc_of = [&](uint32_t s) {
    return reinterpret_cast<const float4*>(ws_acc + (p0 + (size_t)s * n_heads) * IRM_D_LATENT)[threadIdx.x];
  };
  float mx = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float2 m2, float4 v) {
    const float f = (m2.x == -INFINITY) ? 0.f : exp2f(m2.x - mx);
    L += f * m2.y;
    acc.x += f * v.x;
    acc.y += f * v.y;
    acc.z += f * v.z;
    acc.w += f * v.w;
  };
  if constexpr (kMax > 0) {
    float2 m2[kMax];
    float4 v[kMax];
#pragma unroll
    for (int s = 0; s < kMax; ++s) {
      m2[s] = (uint32_t)s < n_parts ? ml[p0 + (size_t)s * n_heads] : make_float2(-INFINITY, 0.f);
      v[s] = (uint32_t)s < n_parts ? acc_of(s) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int s = 0; s < kMax; ++s) mx = fmaxf(mx, m2[s].x);
#pragma unroll
    for (int s = 0; s < kMax; ++s) add(m2[s], v[s]);
  } else {
#pragma unroll 8
    for (uint32_t s = 0; s < n_parts; ++s) mx = fmaxf(mx, ml[p0 + (size_t)s * n_heads].x);
#pragma unroll 8
    for (uint32_t s = 0; s < n_parts; ++s) add(ml[p0 + (size_t)s * n_heads], acc_of(s));
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
  ra.trig = image_of(t).trig;
  ra.pool_last = pool_last_of(pool_rows);
  return ra;
}

}  // namespace

uint32_t decode_default_splits(const irm_table* t, uint32_t n_groups) {
  // one workgroup per CU (256 CUs) with >= 64 rows per split (a 16-row
  // slice for each wave of the 16-head kernel, two 32-row tiles for the
  // shared-tile one); a workgroup covers four head groups when the head count
  // allows it.  Small batches thus get more, shorter splits: the
  // 1-sequence, 1024-row decode takes 17 us in 16 splits against 21.5 us in 4.
  if (t->n_seq == 0 || n_groups == 0) return 1;  // an empty batch has nothing to split
  const uint32_t units = (n_groups % 4 == 0) ? n_groups / 4 : n_groups;
  const uint32_t want = (256 + t->n_seq * units - 1) / (t->n_seq * units);
  const uint32_t cap = (t->max_seq_len + 63) / 64;
  uint32_t s = want < cap ? want : cap;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return s;
}

// Compute units of the current device (cached per thread and device).
static uint32_t cu_count() {
  static thread_local int dev_cached = -1;
  static thread_local uint32_t n_cached = 256;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return n_cached;
  if (dev != dev_cached) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      n_cached = (uint32_t)n;
    dev_cached = dev;
  }
  return n_cached;
}

// Consecutive splits per workgroup of the shared-tile kernel: the largest
// divisor of n_splits that still leaves a workgroup for every compute unit.
static uint32_t splits_per_workgroup(uint32_t n_seq, uint32_t n_splits, uint32_t n_blk) {
  const uint64_t cus = cu_count();
  uint32_t best = 1;
  for (uint32_t u = 2; u <= n_splits; ++u)
    if (n_splits % u == 0 && (uint64_t)n_seq * (n_splits / u) * n_blk >= cus) best = u;
  return best;
}

// Consecutive splits one workgroup streams (1 for the 16-head-group kernel).
static uint32_t splits_per_wg_of(const irm_table* t, uint32_t n_heads, uint32_t n_splits) {
  const uint32_t G = n_heads / 16;
  return G % kSplitGroups == 0 ? splits_per_workgroup(t->n_seq, n_splits, G / kSplitGroups) : 1;
}

uint32_t decode_parts(const irm_table* t, uint32_t n_heads, uint32_t n_splits) {
  return n_splits / splits_per_wg_of(t, n_heads, n_splits);
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
  const bool shared = G % kSplitGroups == 0;
  a.splits_per_wg = splits_per_wg_of(t, n_heads, n_splits);
  const uint64_t bs = (uint64_t)t->n_seq * (n_splits / a.splits_per_wg);
  const uint64_t grid = (bs + 7) / 8 * 8 * (shared ? G / kSplitGroups : G);
  if (grid > 0x7fffffffull) return fail(IRM_EUNSUPPORTED, "irm_mla_decode: grid too large");
  if (shared)
    hipLaunchKernelGGL(decode_shared_kernel, dim3((uint32_t)grid), dim3(kRoleThreads), 0, s, a);
  else
    hipLaunchKernelGGL(decode_private_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, s, a);
  irm_status st = launch_check("irm_mla_decode: split kernel");
  if (st != IRM_OK) return st;
  const uint32_t n_parts = n_splits / a.splits_per_wg;
  const dim3 cgrid(t->n_seq * n_heads), cblock(128);
  uint16_t* o16 = static_cast<uint16_t*>(out);
  if (n_parts <= 4)
    hipLaunchKernelGGL(decode_combine_kernel<4>, cgrid, cblock, 0, s, ws_acc, ws_ml, o16, lse, n_heads, n_parts);
  else if (n_parts <= 16)
    hipLaunchKernelGGL(decode_combine_kernel<16>, cgrid, cblock, 0, s, ws_acc, ws_ml, o16, lse, n_heads, n_parts);
  else
    hipLaunchKernelGGL(decode_combine_kernel<0>, cgrid, cblock, 0, s, ws_acc, ws_ml, o16, lse, n_heads, n_parts);
  return launch_check("irm_mla_decode: combine kernel");
}

irm_status decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  irm_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (st != IRM_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(IRM_EUNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    st = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st != IRM_OK) return st;
    if (!p || reinterpret_cast<uintptr_t>(p) % kAlign)
      return fail(IRM_EHIP, "hipGetSymbolAddress(scratch): no aligned device address");
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return IRM_OK;
}

}  // namespace irm
