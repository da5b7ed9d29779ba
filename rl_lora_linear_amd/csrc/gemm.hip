// bf16 MFMA GEMM for gfx950: C[M][N] = sum_k A[m][k] * B[n][k] (both operands
// K-contiguous, fp32 accumulation), with three epilogues:
//   EPI_BF16  store bf16(C)                                  (base GEMMs, dh)
//   EPI_LSE   per-row (max, sum exp) over the tile's columns and the target
//             logit, for the lm_head online logsumexp        (token_logprobs)
//   EPI_GRAD  G = d (onehot(y) - exp(C - lse)) stored bf16   (logprob backward)
//
// Block tile 256 x 256 x 64, 256 threads = 4 waves in a 2 x 2 grid, each wave
// 128 x 128 as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators
// per lane).  Global -> register -> LDS staging, double-buffered (2 x 64 KB of
// LDS), one barrier per K step; the global loads of step k+1 are issued before
// the MFMAs of step k.  LDS rows are 128 B (64 bf16) and their 16-byte chunks
// are XOR-swizzled by (row & 7), so the 16-byte fragment reads of 8 consecutive
// rows hit distinct banks.  Tiles are ordered XCD-first (blocks are dispatched
// round-robin over the 8 XCDs, so each XCD gets a contiguous tile range and
// its own L2 sees the reuse) and then in groups of `group_m` row tiles.
#include "common.hpp"

namespace lora {

enum { EPI_BF16 = 0, EPI_LSE = 1, EPI_GRAD = 2 };

struct GemmEpi {
  uint16_t* C;            // EPI_BF16 / EPI_GRAD output
  int64_t ldc;
  float* part_m;          // EPI_LSE: [tiles_n][M]
  float* part_s;          // EPI_LSE: [tiles_n][M]
  float* zt;              // EPI_LSE: [M] target logit
  const int32_t* targets; // EPI_LSE / EPI_GRAD: [M]
  const float* lse;       // EPI_GRAD: [M]
  const float* dlogp;     // EPI_GRAD: [M]
};

constexpr int GBM = 256, GBN = 256, GBK = 64;
constexpr int G_CHUNKS = GBK / 8;            // 16-byte chunks per LDS row
constexpr int G_TILE_U4 = GBM * G_CHUNKS;    // uint4 per operand tile
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int lds_idx(int row, int chunk) { return row * G_CHUNKS + (chunk ^ (row & 7)); }

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_nt_kernel(const uint16_t* __restrict__ A,
                                                         const uint16_t* __restrict__ B, int M,
                                                         int N, int K, int64_t lda, int64_t ldb,
                                                         GemmEpi ep, int tiles_m, int tiles_n,
                                                         int group_m) {
  extern __shared__ uint4 smem[];  // [2][A tile] [2][B tile]
  uint4* As = smem;
  uint4* Bs = smem + 2 * G_TILE_U4;

  // ---- tile id: XCD-contiguous, then grouped along M
  const int num = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, loc = bid >> 3;
  const int per = num >> 3, rem = num & 7;
  const int t = (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
  const int gsz = group_m * tiles_n;
  const int grp = t / gsz;
  const int first_m = grp * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int in = t - grp * gsz;
  const int tm = first_m + in % gm;
  const int tn = in / gm;
  const int m0 = tm * GBM, n0 = tn * GBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- global load mapping: 8 threads per 128-byte row, 32 rows per pass
  const int ld_row = tid >> 3, ld_chunk = tid & 7;
  const uint16_t* a_base = A + (int64_t)(m0 + ld_row) * lda + ld_chunk * 8;
  const uint16_t* b_base = B + (int64_t)(n0 + ld_row) * ldb + ld_chunk * 8;
  const int64_t a_step = 32 * lda, b_step = 32 * ldb;
  const int a_lim = M - m0 - ld_row;  // pass i is in range iff 32*i < a_lim
  const int b_lim = N - n0 - ld_row;
  uint4 ra[8], rb[8];

#define GEMM_GLOAD(k0)                                                                 \
  _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                       \
    ra[i] = (32 * i < a_lim) ? *(const uint4*)(a_base + i * a_step + (k0))              \
                             : make_uint4(0, 0, 0, 0);                                  \
    rb[i] = (32 * i < b_lim) ? *(const uint4*)(b_base + i * b_step + (k0))              \
                             : make_uint4(0, 0, 0, 0);                                  \
  }
#define GEMM_SSTORE(buf)                                                               \
  _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                       \
    As[(buf) * G_TILE_U4 + lds_idx(ld_row + 32 * i, ld_chunk)] = ra[i];                 \
    Bs[(buf) * G_TILE_U4 + lds_idx(ld_row + 32 * i, ld_chunk)] = rb[i];                 \
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < 16; ++g) acc[i][j][g] = 0.f;

  const int KT = K / GBK;
  GEMM_GLOAD(0);
  GEMM_SSTORE(0);
  __syncthreads();

  const int frag_row = lane & 31;   // row within a 32-row MFMA tile
  const int frag_half = lane >> 5;  // which 8-wide k half of the 16-wide k slice

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) { GEMM_GLOAD((kt + 1) * GBK); }
    const uint4* At = As + buf * G_TILE_U4;
    const uint4* Bt = Bs + buf * G_TILE_U4;
#pragma unroll
    for (int kk = 0; kk < GBK / 16; ++kk) {
      const int c = 2 * kk + frag_half;
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = as_bf16x8(At[lds_idx(wm * 128 + i * 32 + frag_row, c)]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = as_bf16x8(Bt[lds_idx(wn * 128 + j * 32 + frag_row, c)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < KT) { GEMM_SSTORE(buf ^ 1); }
    __syncthreads();
  }

#undef GEMM_GLOAD
#undef GEMM_SSTORE

  // ---- epilogues.  Accumulator layout of a 32x32 tile: register g of lane l
  // holds row 8*(g/4) + 4*(l/32) + (g%4), column l%32.
  const int col_l = lane & 31;
  const int row_q = 4 * (lane >> 5);

  if constexpr (EPI == EPI_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 128 + j * 32 + col_l;
        if (col >= N) continue;
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          const int row = m0 + wm * 128 + i * 32 + 8 * (g >> 2) + row_q + (g & 3);
          if (row < M) ep.C[(int64_t)row * ep.ldc + col] = f2bf(acc[i][j][g]);
        }
      }
  } else if constexpr (EPI == EPI_LSE) {
    __shared__ int32_t tgt_s[GBM];
    __shared__ float2 red_s[2][GBM];
    for (int r = tid; r < GBM; r += 256) tgt_s[r] = (m0 + r < M) ? ep.targets[m0 + r] : -1;
    __syncthreads();
    const int cbase = n0 + wn * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        const int rl = wm * 128 + i * 32 + 8 * (g >> 2) + row_q + (g & 3);
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (cbase + j * 32 + col_l < N) mx = fmaxf(mx, acc[i][j][g]);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float sm = 0.f;
        if (mx != -INFINITY) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (cbase + j * 32 + col_l < N) sm += exp2f((acc[i][j][g] - mx) * kLog2e);
        }
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) sm += __shfl_xor(sm, o);
        const int y = tgt_s[rl];
        const int yo = y - cbase;
        if (yo >= 0 && yo < 128 && (yo & 31) == col_l && m0 + rl < M) {
          const int jj = yo >> 5;
          float zv = acc[i][0][g];
#pragma unroll
          for (int j = 1; j < 4; ++j)
            if (j == jj) zv = acc[i][j][g];
          if (y < N) ep.zt[m0 + rl] = zv;
        }
        if (col_l == 0) red_s[wn][rl] = make_float2(mx, sm);
      }
    }
    __syncthreads();
    for (int r = tid; r < GBM; r += 256) {
      if (m0 + r >= M) continue;
      float2 a = red_s[0][r], b = red_s[1][r];
      float mx = fmaxf(a.x, b.x);
      float sm = 0.f;
      if (a.x != -INFINITY) sm += a.y * exp2f((a.x - mx) * kLog2e);
      if (b.x != -INFINITY) sm += b.y * exp2f((b.x - mx) * kLog2e);
      ep.part_m[(int64_t)tn * M + m0 + r] = mx;
      ep.part_s[(int64_t)tn * M + m0 + r] = sm;
    }
  } else {  // EPI_GRAD
    __shared__ int32_t tgt_s[GBM];
    __shared__ float lse_s[GBM];
    __shared__ float d_s[GBM];
    for (int r = tid; r < GBM; r += 256) {
      const bool ok = m0 + r < M;
      int y = ok ? ep.targets[m0 + r] : -1;
      float d = ok ? ep.dlogp[m0 + r] : 0.f;
      if (y < 0 || y >= N) d = 0.f;  // invalid target: zero row
      tgt_s[r] = y;
      lse_s[r] = ok ? ep.lse[m0 + r] : 0.f;
      d_s[r] = d;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        const int rl = wm * 128 + i * 32 + 8 * (g >> 2) + row_q + (g & 3);
        if (m0 + rl >= M) continue;
        const float d = d_s[rl], l = lse_s[rl];
        const int y = tgt_s[rl];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + wn * 128 + j * 32 + col_l;
          if (col >= N) continue;
          float gv = 0.f;
          if (d != 0.f) {
            const float p = exp2f((acc[i][j][g] - l) * kLog2e);
            gv = d * ((col == y ? 1.f : 0.f) - p);
          }
          ep.C[(int64_t)(m0 + rl) * ep.ldc + col] = f2bf(gv);
        }
      }
  }
}

}  // namespace lora

namespace lora_host {

using namespace lora;

static int pick_group_m(int tiles_m) { return tiles_m < 8 ? tiles_m : 8; }

template <int EPI>
static lora_status launch_gemm(const uint16_t* A, const uint16_t* B, int M, int N, int K,
                               int64_t lda, int64_t ldb, const GemmEpi& ep, hipStream_t s,
                               int group_m) {
  if (M <= 0 || N <= 0) return LORA_OK;
  const int tiles_m = (int)cdiv(M, GBM), tiles_n = (int)cdiv(N, GBN);
  if (group_m <= 0) group_m = pick_group_m(tiles_m);
  if (group_m > tiles_m) group_m = tiles_m;
  const size_t lds = 4 * G_TILE_U4 * sizeof(uint4);
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)gemm_nt_kernel<EPI>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr_set = true;
  }
  hipLaunchKernelGGL(gemm_nt_kernel<EPI>, dim3(tiles_m * tiles_n), dim3(256), lds, s, A, B, M, N,
                     K, lda, ldb, ep, tiles_m, tiles_n, group_m);
  return launch_check("gemm_nt");
}

lora_status gemm_nt_bf16(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                         int64_t lda, int64_t ldb, int64_t ldc, hipStream_t s, int group_m) {
  GemmEpi ep{};
  ep.C = C;
  ep.ldc = ldc;
  return launch_gemm<EPI_BF16>(A, B, M, N, K, lda, ldb, ep, s, group_m);
}

lora_status gemm_nt_lse(const uint16_t* A, const uint16_t* B, int M, int N, int K, int64_t lda,
                        int64_t ldb, float* part_m, float* part_s, float* zt,
                        const int32_t* targets, hipStream_t s, int group_m) {
  GemmEpi ep{};
  ep.part_m = part_m;
  ep.part_s = part_s;
  ep.zt = zt;
  ep.targets = targets;
  return launch_gemm<EPI_LSE>(A, B, M, N, K, lda, ldb, ep, s, group_m);
}

lora_status gemm_nt_grad(const uint16_t* A, const uint16_t* B, uint16_t* G, int64_t ldg, int M,
                         int N, int K, int64_t lda, int64_t ldb, const int32_t* targets,
                         const float* lse, const float* dlogp, hipStream_t s, int group_m) {
  GemmEpi ep{};
  ep.C = G;
  ep.ldc = ldg;
  ep.targets = targets;
  ep.lse = lse;
  ep.dlogp = dlogp;
  return launch_gemm<EPI_GRAD>(A, B, M, N, K, lda, ldb, ep, s, group_m);
}

}  // namespace lora_host
