// bf16 projections on the matrix cores for gfx950: Y_g = A_g . W_g^T for
// g < groups, bf16 operands, f32 accumulation, bf16 result (the precision
// paragraph of the "deepseek_v41_ref::attn" rustdoc: every projection is
// linear_bf16).  With groups > 1 this is the block-diagonal wo_a of the
// "Grouped output" step of the "Compressed sparse attention" page (each group
// of heads contracted with its own block), with groups == 1 the plain wo_b.
//
// Tiles: a workgroup of four wavefronts (2 x 2) owns a BM x BN block of Y and
// walks K in stages of 64: the A and W stages go global -> registers -> LDS
// (rows padded to 144 bytes, so the 16 rows one MFMA operand read touches
// fall on distinct banks), double-buffered with the next stage's loads in
// flight during the products; one barrier per stage.  Products are
// v_mfma_f32_16x16x32_bf16 with A rows as the M operand and W rows (the
// output features) as the N operand.
//
// Few rows (a decode step's tokens) make the weights the whole cost: K is
// then split over workgroups, each writing f32 partial sums that a second
// kernel adds in a fixed order (so the result does not depend on timing).
// Workgroups that share an A slice are placed on one XCD (dispatch is
// round-robin over the 8 XCDs), so the slice is read from HBM once per XCD.
#include "v41_common.h"
#include "v41_gemm.h"

namespace v41 {
namespace {

constexpr int kBK = 64;
constexpr int kRowBytes = kBK * 2 + 16;
constexpr int kGemmThreads = 256;

struct GemmParams {
  const uint16_t* a;
  int64_t lda, a_gs;
  const uint16_t* w;
  int64_t ldw, w_gs;
  uint16_t* y;
  int64_t ldy, y_gs;
  float* part;
  int32_t M, N, K, groups, splits, kc;
  int32_t m_tiles, n_tiles;
};

template <int BM, int BN>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmParams p) {
  constexpr int TM = BM / 32;          // 16-row tiles per wavefront along M
  constexpr int TN = BN / 32;          // along N
  constexpr int kAChunks = BM * 8 / kGemmThreads;
  constexpr int kWChunks = BN * 8 / kGemmThreads;
  constexpr int kStageBytes = (BM + BN) * kRowBytes;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];

  // ---- tile of this workgroup: XCD-chunked order (gs, m tile, n tile)
  const int32_t tiles = p.m_tiles * p.n_tiles;
  const int32_t nwg = p.groups * p.splits * tiles;
  int32_t id = (int32_t)blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int32_t gs = id / tiles;
  const int32_t rem = id - gs * tiles;
  const int32_t mt = rem / p.n_tiles;
  const int32_t nt = rem - mt * p.n_tiles;
  const int32_t g = gs / p.splits;
  const int32_t sp = gs - g * p.splits;
  const int32_t m0 = mt * BM, n0 = nt * BN;
  const int32_t k_begin = sp * p.kc;
  const int32_t k_end = min(p.K, k_begin + p.kc);
  const int32_t n_stages = (k_end - k_begin) / kBK;

  const uint16_t* __restrict__ A = p.a + g * p.a_gs;
  const uint16_t* __restrict__ W = p.w + g * p.w_gs;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- this thread's 16-byte chunks of a stage
  u32x4 ra[kAChunks], rw[kWChunks];
  auto load_stage = [&](int32_t k0) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int c = tid + kGemmThreads * i;
      const int r = c >> 3, c16 = c & 7;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m0 + r < p.M)
        v = *reinterpret_cast<const u32x4*>(A + (int64_t)(m0 + r) * p.lda + k0 + 8 * c16);
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < kWChunks; ++i) {
      const int c = tid + kGemmThreads * i;
      const int r = c >> 3, c16 = c & 7;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (n0 + r < p.N)
        v = *reinterpret_cast<const u32x4*>(W + (int64_t)(n0 + r) * p.ldw + k0 + 8 * c16);
      rw[i] = v;
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* st = smem + buf * kStageBytes;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int c = tid + kGemmThreads * i;
      *reinterpret_cast<u32x4*>(st + (c >> 3) * kRowBytes + 16 * (c & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < kWChunks; ++i) {
      const int c = tid + kGemmThreads * i;
      *reinterpret_cast<u32x4*>(st + (BM + (c >> 3)) * kRowBytes + 16 * (c & 7)) = rw[i];
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // lane's operand offsets inside a stage: row lane%16 of each 16-row tile,
  // 16-byte k group lane/16
  const int a_off = (wm * (BM / 2) + (lane & 15)) * kRowBytes + 16 * (lane >> 4);
  const int w_off = (BM + wn * (BN / 2) + (lane & 15)) * kRowBytes + 16 * (lane >> 4);

  if (n_stages > 0) {
    load_stage(k_begin);
    store_stage(0);
  }
  __syncthreads();
  for (int32_t s = 0; s < n_stages; ++s) {
    const int buf = s & 1;
    if (s + 1 < n_stages) load_stage(k_begin + (s + 1) * kBK);
    const uint8_t* base = smem + buf * kStageBytes;
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      bf16x8 af[TM], wf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = as_bf16x8(
            *reinterpret_cast<const u32x4*>(base + a_off + i * 16 * kRowBytes + ks * 64));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        wf[j] = as_bf16x8(
            *reinterpret_cast<const u32x4*>(base + w_off + j * 16 * kRowBytes + ks * 64));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32(af[i], wf[j], acc[i][j]);
    }
    if (s + 1 < n_stages) store_stage(buf ^ 1);
    __syncthreads();
  }

  // ---- results: lane holds rows 4*(lane/16) + 0..3 and column lane%16 of
  // each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int32_t n = n0 + wn * (BN / 2) + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int32_t m = m0 + wm * (BM / 2) + i * 16 + 4 * (lane >> 4) + e;
        if (m < p.M && n < p.N) {
          if (p.splits == 1) {
            p.y[g * p.y_gs + (int64_t)m * p.ldy + n] = (uint16_t)f32_to_bf16_bits(acc[i][j][e]);
          } else {
            p.part[(((int64_t)sp * p.groups + g) * p.M + m) * p.N + n] = acc[i][j][e];
          }
        }
      }
    }
  }
}

// y = bf16(sum over splits of the partials), splits added in index order.
// One thread per 4 consecutive outputs of a row (N a multiple of 4): 16-byte
// partial loads, all splits issued before the adds, one 8-byte store.
__global__ __launch_bounds__(256) void gemm_reduce4_kernel(const float* __restrict__ part,
                                                           int32_t splits, int32_t rows,
                                                           int32_t M, int32_t N, uint16_t* y,
                                                           int64_t ldy, int64_t y_gs) {
  const int32_t q = N / 4;  // quads per row
  const int64_t per_split = (int64_t)rows * N;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // quad index
  if (e >= (int64_t)rows * q) return;
  const int64_t row = e / q;                 // g * M + m
  const int32_t n = (int32_t)(e - row * q) * 4;
  const float* src = part + row * N + n;
  f32x4 acc = *reinterpret_cast<const f32x4*>(src);
  for (int32_t k = 1; k < splits; ++k) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + k * per_split);
    acc[0] += v[0];
    acc[1] += v[1];
    acc[2] += v[2];
    acc[3] += v[3];
  }
  const int64_t g = row / M, m = row - g * M;
  uint2 o;
  o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
  o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
  uint16_t* dst = y + g * y_gs + m * ldy + n;
  if ((reinterpret_cast<uintptr_t>(dst) & 7u) == 0) {
    *reinterpret_cast<uint2*>(dst) = o;
  } else {
    dst[0] = (uint16_t)(o.x & 0xFFFFu);
    dst[1] = (uint16_t)(o.x >> 16);
    dst[2] = (uint16_t)(o.y & 0xFFFFu);
    dst[3] = (uint16_t)(o.y >> 16);
  }
}

// The same for any N, one output per thread.
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ part,
                                                          int32_t splits, int32_t groups,
                                                          int32_t M, int32_t N, uint16_t* y,
                                                          int64_t ldy, int64_t y_gs) {
  const int64_t per_split = (int64_t)groups * M * N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < per_split; e += stride) {
    float s = 0.f;
    for (int32_t k = 0; k < splits; ++k) s += part[k * per_split + e];
    const int64_t g = e / ((int64_t)M * N);
    const int64_t r = e - g * M * N;
    const int64_t m = r / N, n = r - m * N;
    y[g * y_gs + m * ldy + n] = (uint16_t)f32_to_bf16_bits(s);
  }
}

}  // namespace

int gemm_splits(int32_t M, int32_t N, int32_t K, int32_t groups) {
  // few rows: split K until about 512 workgroups, each with >= 512 of K
  if (M > 64) return 1;
  const int64_t tiles = (int64_t)groups * ((N + 63) / 64);
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t max_s = K / 512;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  if (s > 16) s = 16;
  return (int)s;
}

int64_t gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t groups) {
  const int s = gemm_splits(M, N, K, groups);
  return s > 1 ? (int64_t)s * groups * M * N * 4 : 0;
}

hipError_t launch_linear_bf16(const LinearArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0 || a.groups == 0) return hipSuccess;
  int splits = gemm_splits(a.M, a.N, a.K, a.groups);
  while (splits > 1 && (a.workspace == nullptr ||
                        (int64_t)splits * a.groups * a.M * a.N * 4 > a.workspace_bytes))
    --splits;
  GemmParams p;
  p.a = a.a;
  p.lda = a.lda;
  p.a_gs = a.a_gs;
  p.w = a.w;
  p.ldw = a.ldw;
  p.w_gs = a.w_gs;
  p.y = a.y;
  p.ldy = a.ldy;
  p.y_gs = a.y_gs;
  p.part = splits > 1 ? reinterpret_cast<float*>(a.workspace) : nullptr;
  p.M = a.M;
  p.N = a.N;
  p.K = a.K;
  p.groups = a.groups;
  // K per split, whole stages
  const int32_t stages = a.K / kBK;
  const int32_t per = (stages + splits - 1) / splits;
  p.kc = per * kBK;
  p.splits = (stages + per - 1) / per;
  const bool small = a.M <= 64;
  const int bm = small ? 64 : 128, bn = small ? 64 : 128;
  p.m_tiles = (a.M + bm - 1) / bm;
  p.n_tiles = (a.N + bn - 1) / bn;
  const int64_t nwg = (int64_t)p.groups * p.splits * p.m_tiles * p.n_tiles;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (small)
    hipLaunchKernelGGL((gemm_kernel<64, 64>), dim3((unsigned)nwg), dim3(kGemmThreads), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_kernel<128, 128>), dim3((unsigned)nwg), dim3(kGemmThreads), 0, s,
                       p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t n = (int64_t)p.groups * p.M * p.N;
  if (p.N % 4 == 0 && n / 4 <= 0x7FFFFFFFLL * 256) {
    const int64_t blocks = (n / 4 + 255) / 256;
    hipLaunchKernelGGL(gemm_reduce4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p.part,
                       p.splits, p.groups * p.M, p.M, p.N, a.y, a.ldy, a.y_gs);
  } else {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p.part,
                       p.splits, p.groups, p.M, p.N, a.y, a.ldy, a.y_gs);
  }
  return hipGetLastError();
}

}  // namespace v41
