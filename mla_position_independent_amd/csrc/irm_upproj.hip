// Non-absorbed MLA prefill, up-projection: the latent rows of an assembled
// cache become a full key and value per head, kvh[h][t] = [W_UK[h] c_KV[t] |
// W_UV[h] c_KV[t]] (bf16, 256 per row and head) (Irminsul pages:
// gentlecold.top article, section 4 for the key and value from c_KV; section
// 13 for the non-absorbed form, which has to up-project c_KV at run time): a
// [rows x 512] by [512 x 256] product per head on v_mfma_f32_16x16x32_bf16,
// both operands staged through LDS.  Its own source so that it keeps the
// compiler's default scheduling (the attention kernel's file uses another).

#include <hip/hip_runtime.h>

#include "irm_attn.h"
#include "irm_internal.h"
#include "irm_launch.h"

namespace irm {
namespace {

using namespace irm::dev;

// LDS offset of 16-byte unit u of row r in a tile of 128-byte rows: units
// are permuted by (r >> 1) & 7, so 16 lanes reading one unit of 16
// consecutive rows cover all 64 banks.
__device__ __forceinline__ uint32_t pos128(uint32_t r, uint32_t u) { return r * 128 + ((u ^ ((r >> 1) & 7)) << 4); }

// ---------------------------------------------------------------------------
// up-projection
//
// Workgroup = (head h, 64 rows), four waves, two workgroups per compute unit
// (each 80 KB of LDS; measured 15% faster than one workgroup of 128 rows,
// whose chunk copies each wave then waited for); wave w computes features
// 64w .. 64w+63 of the head's 256 (waves 0-1: W_UK, 2-3: W_UV) for all 64
// rows, as D = W A^T: lane (q, r) ends with features 4q..4q+3 of a 16-feature
// block for row r of a 16-row block, stored as 8 bytes.  The latent
// dimension goes in 64-wide chunks through two LDS stages (kv rows 64 x 128
// B, weights 256 x 128 B); within a chunk, MFMA step s takes units 4s + q.
// ---------------------------------------------------------------------------
constexpr int kUpRows = 64;
constexpr int kUpMb = kUpRows / 16;                     // 16-row blocks per workgroup
constexpr int kUpFeat = 256;
constexpr int kUpChunk = 64;                             // latent dims per stage
constexpr int kUpChunks = IRM_D_LATENT / kUpChunk;      // 8
constexpr int kUpA = kUpRows * 128;                      // 8 KB
constexpr int kUpW = kUpFeat * 128;                      // 32 KB

struct UpSmem {
  unsigned char a[2][kUpA];
  unsigned char w[2][kUpW];
};

static_assert(2 * sizeof(UpSmem) <= 160 * 1024, "two workgroups per compute unit fit the LDS");

struct UpArgs {
  const unsigned char* kv;     // bf16 [rows][576]
  const unsigned char* w_uk;   // bf16 [H][128][512]
  const unsigned char* w_uv;   // bf16 [H][128][512]
  unsigned char* out;          // bf16 [H][rows][256]
  uint32_t rows, n_heads, row_tiles;
};

// Copies of chunk c into stage st: wave w moves kv rows 16w .. 16w+15 (2 KB)
// and weight rows 64w .. 64w+63 (8 KB); lane l of a 1 KB copy fills row
// base + l / 8, LDS position l % 8.
__device__ __forceinline__ void up_issue(const UpArgs& a, UpSmem& sm, int st, uint32_t h, uint32_t m0, int c) {
  const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t p = lane & 7;
#pragma unroll
  for (int i = 0; i < kUpRows / 32; ++i) {
    const uint32_t r = (kUpRows / 4) * w + 8 * i + (lane >> 3);
    const uint32_t u = p ^ ((r >> 1) & 7);
    const uint32_t row = min(m0 + r, a.rows - 1);
    dma16(a.kv + (size_t)row * kRowBytes + c * 128 + 16 * u, lds_addr(sm.a[st] + ((kUpRows / 4) * w + 8 * i) * 128));
  }
  const unsigned char* wsrc = (w < 2 ? a.w_uk : a.w_uv) + (size_t)h * 128 * IRM_D_LATENT * 2;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t f = 64 * w + 8 * i + (lane >> 3);  // feature of the head, 0..255
    const uint32_t u = p ^ ((f >> 1) & 7);
    dma16(wsrc + (size_t)(f & 127) * IRM_D_LATENT * 2 + c * 128 + 16 * u,
          lds_addr(sm.w[st] + (64 * w + 8 * i) * 128));
  }
}

__global__ __launch_bounds__(kThreads, 2) void upproj_kernel(UpArgs a) {
  __shared__ UpSmem sm;
  const uint32_t b = blockIdx.x;
  const uint32_t h = b % a.n_heads, m0 = (b / a.n_heads) * kUpRows;
  const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t q = lane >> 4, r = lane & 15;

  f32x4_t acc[4][kUpMb];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < kUpMb; ++mb) acc[nb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  up_issue(a, sm, 0, h, m0, 0);
  for (int c = 0; c < kUpChunks; ++c) {
    const int st = c & 1;
    wait_dma_all();
    __syncthreads();  // chunk c is in LDS; every wave is done with chunk c - 1
    if (c + 1 < kUpChunks) up_issue(a, sm, st ^ 1, h, m0, c + 1);
    const unsigned char* A = sm.a[st];
    const unsigned char* W = sm.w[st];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t u = 4 * s + q;
      bf16x8_t wf[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        wf[nb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(W + pos128(64 * w + 16 * nb + r, u)));
#pragma unroll
      for (int mb = 0; mb < kUpMb; ++mb) {
        const bf16x8_t af = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(A + pos128(16 * mb + r, u)));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[nb], af, acc[nb][mb], 0, 0, 0);
      }
    }
  }
  // lane (q, r): features 64w + 16nb + 4q .. +3 of row m0 + 16mb + r
#pragma unroll
  for (int mb = 0; mb < kUpMb; ++mb) {
    const uint32_t m = m0 + 16 * mb + r;
    if (m >= a.rows) continue;
    unsigned char* dst = a.out + ((size_t)h * a.rows + m) * (kUpFeat * 2) + (64 * w + 4 * q) * 2;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const f32x4_t& v = acc[nb][mb];
      *reinterpret_cast<uint2*>(dst + 32 * nb) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
    }
  }
}

}  // namespace

irm_status launch_kv_upproj(const void* kv, uint64_t kv_rows, const void* w_uk, const void* w_uv, uint32_t n_heads,
                            void* out, hipStream_t s) {
  if (!kv_rows) return IRM_OK;
  UpArgs a;
  a.kv = static_cast<const unsigned char*>(kv);
  a.w_uk = static_cast<const unsigned char*>(w_uk);
  a.w_uv = static_cast<const unsigned char*>(w_uv);
  a.out = static_cast<unsigned char*>(out);
  a.rows = (uint32_t)kv_rows;
  a.n_heads = n_heads;
  const uint64_t tiles = (kv_rows + kUpRows - 1) / kUpRows, grid = tiles * n_heads;
  if (grid * kThreads > 0xffffffffull) return fail(IRM_EUNSUPPORTED, "irm_mla_kv_upproj: grid too large");
  a.row_tiles = (uint32_t)tiles;
  hipLaunchKernelGGL(upproj_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, s, a);
  return launch_check("up-projection kernel");
}

}  // namespace irm
