// Bandwidth-bound kernels of the hot path on gfx950: the logsumexp merge, the
// token loss, per-adapter AdamW, the SwiGLU glue, and a bf16 transpose for
// keeping frozen operands in both layouts.
#include <vector>

#include "common.hpp"
#include "sgmv.hpp"

namespace lora {

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;

// ------------------------------------------------------------------ logsumexp merge
// Merge of the per-vocab-tile (max, sum) pairs (TPU RL note, section 10 item 3:
// lse = m + log sum exp(z - m)), then logprob = z[target] - lse.  Out-of-range
// targets give NaN and a status flag.
// A block owns 64 tokens (one per lane, so every load is 256 contiguous bytes)
// and its 16 waves split the vocab tiles: wave w folds tiles w, w + 16, ... in
// that order with the running rescale m' = max(m, m_i), s' = s e^(m - m') +
// s_i e^(m_i - m'), eight tiles' loads in flight at a time; the 16 wave results
// are folded the same way in wave order.  (One thread per token over all the
// tiles left the chip nearly idle: 64 blocks for 16384 tokens.)
constexpr int MERGE_WAVES = 16;
constexpr int MERGE_BATCH = 8;

__device__ __forceinline__ void lse_fold(float& mx, float& s, float m, float si) {
  if (m > mx) {
    s = s * exp2f((mx - m) * kLog2eF) + si;   // mx = -inf: s is still 0
    mx = m;
  } else if (m != -INFINITY) {
    s += si * exp2f((m - mx) * kLog2eF);
  }
}

__global__ __launch_bounds__(64 * MERGE_WAVES) void logprob_merge_kernel(
    const float* __restrict__ part_m, const float* __restrict__ part_s,
    const float* __restrict__ zt, const int32_t* __restrict__ targets, int64_t n, int tiles,
    int64_t vocab, float* __restrict__ logprobs, float* __restrict__ lse, int32_t* status) {
  __shared__ float s_m[MERGE_WAVES][64], s_s[MERGE_WAVES][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 64 + lane;
  float mx = -INFINITY, s = 0.f;
  if (t < n) {
    for (int i0 = w; i0 < tiles; i0 += MERGE_BATCH * MERGE_WAVES) {
      float mm[MERGE_BATCH], ss[MERGE_BATCH];
#pragma unroll
      for (int u = 0; u < MERGE_BATCH; ++u) {
        const int i = i0 + u * MERGE_WAVES;
        mm[u] = i < tiles ? part_m[(int64_t)i * n + t] : -INFINITY;
        ss[u] = i < tiles ? part_s[(int64_t)i * n + t] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < MERGE_BATCH; ++u) lse_fold(mx, s, mm[u], ss[u]);
    }
  }
  s_m[w][lane] = mx;
  s_s[w][lane] = s;
  __syncthreads();
  if (w != 0 || t >= n) return;
  mx = -INFINITY;
  s = 0.f;
  for (int v = 0; v < MERGE_WAVES; ++v) lse_fold(mx, s, s_m[v][lane], s_s[v][lane]);
  const float l = mx + log2f(s) * kLn2F;
  lse[t] = l;
  const int32_t y = targets[t];
  if (y < 0 || y >= vocab) {
    set_flag(status, LORA_FLAG_TARGET_RANGE);
    logprobs[t] = __int_as_float(0x7FC00000);
  } else {
    logprobs[t] = zt[t] - l;
  }
}

// ------------------------------------------------------------------ token loss
// 1024 rows per block (4 per thread); the block's loss terms are summed in
// fp64 by a fixed tree; a second single-block pass sums the block partials in
// block order.  The result depends only on n and the inputs.
// Rows are kept where the weight / mask is non-zero.  A kept row whose own
// inputs to its loss term are not all finite (l, and w, A, l_sampler or g as
// the kind reads them) is removed by selection like a masked row and raises
// LORA_FLAG_NONFINITE_LOSS (TPU RL note, section 12: NaN-logprob sentinel,
// weight zeroed and value neutralised).
constexpr int LOSS_ROWS = 1024;

__device__ __forceinline__ bool fin(float x) { return __builtin_isfinite(x); }

__global__ __launch_bounds__(256) void loss_rows_kernel(int kind, int64_t n,
                                                        const float* __restrict__ logp,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ adv,
                                                        const float* __restrict__ samp,
                                                        const float* __restrict__ g, float clip_lo,
                                                        float clip_hi, double* __restrict__ partial,
                                                        float* __restrict__ dlogp,
                                                        int32_t* __restrict__ status) {
  __shared__ double red[256];
  double acc = 0.0;
  bool sentinel = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = (int64_t)blockIdx.x * LOSS_ROWS + q * 256 + threadIdx.x;
    if (t >= n) continue;
    const float wt = w[t];
    float d = 0.f;
    double term = 0.0;
    if (wt != 0.f) {  // masked rows are removed by selection
      const float l = logp[t];
      if (kind == LOSS_CROSS_ENTROPY) {
        if (fin(l) && fin(wt)) {
          d = -wt;
          term = -(double)wt * (double)l;
        } else {
          sentinel = true;
        }
      } else if (kind == LOSS_CUSTOM) {
        const float gg = g[t];
        if (fin(l) && fin(wt) && fin(gg)) {
          d = gg;
          term = (double)gg * (double)l;
        } else {
          sentinel = true;
        }
      } else {
        const float A = adv[t], ls = samp[t];
        if (fin(l) && fin(wt) && fin(A) && fin(ls)) {
          const float rho = exp2f((l - ls) * kLog2eF);
          const float ra = rho * A;
          if (kind == LOSS_IMPORTANCE_SAMPLING) {
            d = -ra;
            term = -(double)ra;
          } else {
            const float lo = 1.f - clip_lo, hi = 1.f + clip_hi;
            const float rc = fminf(fmaxf(rho, lo), hi);
            const float obj = fminf(ra, rc * A);
            const bool inactive = (A > 0.f && rho > hi) || (A < 0.f && rho < lo);
            d = inactive ? 0.f : -ra;
            term = -(double)obj;
          }
        } else {
          sentinel = true;
        }
      }
    }
    dlogp[t] = d;
    acc += term;
  }
  if (__any(sentinel) && (threadIdx.x & 63) == 0) set_flag(status, LORA_FLAG_NONFINITE_LOSS);
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void loss_sum_kernel(const double* __restrict__ partial,
                                                       int nb, float* __restrict__ loss_out) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int i = threadIdx.x; i < nb; i += 256) acc += partial[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss_out[0] = (float)red[0];
}

// ------------------------------------------------------------------ AdamW
// One adapter's update is all or nothing (TPU RL note, section 12: a
// non-finite optimizer update is skipped outright).  Three launches: clear the
// per-segment skip flags, scan each segment's gradient for NaN/Inf (any block
// that sees one sets its segment's flag and the status word), then update
// every segment whose flag is clear.  The scan costs one extra read of g
// (4 of the 34 bytes moved per parameter).
__device__ __forceinline__ void adam_one(float& p, float g, float& m, float& v, float lr,
                                         float b1, float b2, float eps, float wd, float step_size,
                                         float inv_sqrt_bc2) {
  m = b1 * m + (1.f - b1) * g;
  v = b2 * v + (1.f - b2) * g * g;
  p = p - lr * wd * p;
  const float denom = __fsqrt_rn(v) * inv_sqrt_bc2 + eps;
  p = p - step_size * __fdiv_rn(m, denom);
}

// Up to ADAM_SEGS segments per launch, described in the kernel arguments.
// Block b belongs to the segment whose block range holds it; each block covers
// 4 x 256 x 4 elements with float4 vectors (scalar path if a segment is not
// 16-byte aligned).
constexpr int ADAM_SEGS = 64;
constexpr int ADAM_BLOCK_ELEMS = 4096;
struct AdamSegs {
  int64_t off[ADAM_SEGS];
  int64_t cnt[ADAM_SEGS];
  int32_t blk0[ADAM_SEGS + 1];
  float step_size[ADAM_SEGS];
  float inv_sqrt_bc2[ADAM_SEGS];
  int32_t n;
  int32_t seg0;   // index of segment 0 of this launch in the caller's list (flag slot)
};

__device__ __forceinline__ int adam_seg_of(const AdamSegs& sg, int b) {
  int s = 0;
  while (s + 1 < sg.n && sg.blk0[s + 1] <= b) ++s;
  return s;
}

__global__ __launch_bounds__(256) void adam_check_kernel(AdamSegs sg, const float* __restrict__ g,
                                                         int32_t* __restrict__ skip,
                                                         int32_t* __restrict__ status) {
  const int b = blockIdx.x;
  const int s = adam_seg_of(sg, b);
  const int64_t base = sg.off[s];
  const int64_t n = sg.cnt[s];
  const int64_t e0 = (int64_t)(b - sg.blk0[s]) * ADAM_BLOCK_ELEMS;
  bool bad = false;
  if (((base & 3) == 0) && ((uintptr_t)g % 16 == 0)) {
#pragma unroll
    for (int q = 0; q < ADAM_BLOCK_ELEMS / 1024; ++q) {
      const int64_t e = e0 + ((int64_t)q * 256 + threadIdx.x) * 4;
      if (e + 4 <= n) {
        const float4 gg = ((const float4*)(g + base))[e / 4];
        bad |= !__builtin_isfinite(gg.x) || !__builtin_isfinite(gg.y) ||
               !__builtin_isfinite(gg.z) || !__builtin_isfinite(gg.w);
      } else {
        for (int64_t k = e; k < n && k < e + 4; ++k) bad |= !__builtin_isfinite(g[base + k]);
      }
    }
  } else {
    for (int64_t k = e0 + threadIdx.x; k < min(n, e0 + ADAM_BLOCK_ELEMS); k += 256)
      bad |= !__builtin_isfinite(g[base + k]);
  }
  // one store per wave that saw a bad element (every writer stores the same 1)
  if (__any(bad) && (threadIdx.x & 63) == 0) {
    skip[sg.seg0 + s] = 1;
    if (status) set_flag(status, LORA_FLAG_NONFINITE_GRAD);
  }
}

__global__ __launch_bounds__(256) void adam_multi_kernel(AdamSegs sg, float* __restrict__ p,
                                                         const float* __restrict__ g,
                                                         float* __restrict__ m,
                                                         float* __restrict__ v, float lr, float b1,
                                                         float b2, float eps, float wd,
                                                         uint16_t* __restrict__ pb,
                                                         const int32_t* __restrict__ skip) {
  const int b = blockIdx.x;
  const int s = adam_seg_of(sg, b);
  if (skip[sg.seg0 + s]) return;   // block-uniform: this adapter's update is skipped
  const int64_t base = sg.off[s];
  const int64_t n = sg.cnt[s];
  const float ss = sg.step_size[s], ib = sg.inv_sqrt_bc2[s];
  const int64_t e0 = (int64_t)(b - sg.blk0[s]) * ADAM_BLOCK_ELEMS;
  const bool vec = ((base & 3) == 0) && (((uintptr_t)p | (uintptr_t)g | (uintptr_t)m | (uintptr_t)v) % 16 == 0);
  if (vec) {
#pragma unroll
    for (int q = 0; q < ADAM_BLOCK_ELEMS / 1024; ++q) {
      const int64_t e = e0 + ((int64_t)q * 256 + threadIdx.x) * 4;
      if (e + 4 <= n) {
        const int64_t i = (base + e) / 4;
        float4 pp = ((float4*)p)[i], mm = ((float4*)m)[i], vv = ((float4*)v)[i];
        const float4 gg = ((const float4*)g)[i];
        adam_one(pp.x, gg.x, mm.x, vv.x, lr, b1, b2, eps, wd, ss, ib);
        adam_one(pp.y, gg.y, mm.y, vv.y, lr, b1, b2, eps, wd, ss, ib);
        adam_one(pp.z, gg.z, mm.z, vv.z, lr, b1, b2, eps, wd, ss, ib);
        adam_one(pp.w, gg.w, mm.w, vv.w, lr, b1, b2, eps, wd, ss, ib);
        ((float4*)p)[i] = pp;
        ((float4*)m)[i] = mm;
        ((float4*)v)[i] = vv;
        if (pb) {
          if ((((uintptr_t)(pb + base + e)) & 7) == 0) {
            *(uint2*)(pb + base + e) = make_uint2(pack2bf(pp.x, pp.y), pack2bf(pp.z, pp.w));
          } else {
            pb[base + e] = f2bf(pp.x); pb[base + e + 1] = f2bf(pp.y);
            pb[base + e + 2] = f2bf(pp.z); pb[base + e + 3] = f2bf(pp.w);
          }
        }
      } else {
        for (int64_t k = e; k < n && k < e + 4; ++k) {
          float pp = p[base + k], mm = m[base + k], vv = v[base + k];
          adam_one(pp, g[base + k], mm, vv, lr, b1, b2, eps, wd, ss, ib);
          p[base + k] = pp; m[base + k] = mm; v[base + k] = vv;
          if (pb) pb[base + k] = f2bf(pp);
        }
      }
    }
  } else {
    for (int64_t k = e0 + threadIdx.x; k < min(n, e0 + ADAM_BLOCK_ELEMS); k += 256) {
      float pp = p[base + k], mm = m[base + k], vv = v[base + k];
      adam_one(pp, g[base + k], mm, vv, lr, b1, b2, eps, wd, ss, ib);
      p[base + k] = pp; m[base + k] = mm; v[base + k] = vv;
      if (pb) pb[base + k] = f2bf(pp);
    }
  }
}

// ------------------------------------------------------------------ SwiGLU

template <bool BWD>
__global__ __launch_bounds__(256) void swiglu_kernel(int64_t n, const uint16_t* __restrict__ dh,
                                                     const uint16_t* __restrict__ gt,
                                                     const uint16_t* __restrict__ up,
                                                     uint16_t* __restrict__ o1,
                                                     uint16_t* __restrict__ o2) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n8 = n / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8 + (n % 8 ? 1 : 0);
       i += stride) {
    const bool full = i < n8;
    const int64_t o = i * 8;
    uint16_t G[8], U[8], D[8];
    if (full) {
      const uint4 a = *(const uint4*)(gt + o), b = *(const uint4*)(up + o);
      const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        G[q] = (uint16_t)(wa[q >> 1] >> ((q & 1) * 16));
        U[q] = (uint16_t)(wb[q >> 1] >> ((q & 1) * 16));
      }
      if (BWD) {
        const uint4 c = *(const uint4*)(dh + o);
        const uint32_t wc[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) D[q] = (uint16_t)(wc[q >> 1] >> ((q & 1) * 16));
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t e = i * 8 + q;
        G[q] = e < n ? gt[e] : 0;
        U[q] = e < n ? up[e] : 0;
        D[q] = (BWD && e < n) ? dh[e] : 0;
      }
    }
    uint16_t r1[8], r2[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (!BWD) r1[q] = swiglu_fwd1(G[q], U[q]);
      else swiglu_bwd1(D[q], G[q], U[q], r1[q], r2[q]);
    }
    if (full) {
      *(uint4*)(o1 + o) = make_uint4(r1[0] | (r1[1] << 16), r1[2] | (r1[3] << 16), r1[4] | (r1[5] << 16), r1[6] | (r1[7] << 16));
      if (BWD)
        *(uint4*)(o2 + o) = make_uint4(r2[0] | (r2[1] << 16), r2[2] | (r2[3] << 16), r2[4] | (r2[5] << 16), r2[6] | (r2[7] << 16));
    } else {
      for (int q = 0; q < 8; ++q) {
        const int64_t e = i * 8 + q;
        if (e < n) {
          o1[e] = r1[q];
          if (BWD) o2[e] = r2[q];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ transpose
// dst[c][r] = src[r][c]; 64 x 64 tiles through LDS (padded to avoid conflicts).
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                             uint16_t* __restrict__ dst,
                                                             int64_t rows, int64_t cols) {
  __shared__ uint16_t tile[64][64 + 2];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) tile[i][tx] = src[(r0 + i) * cols + c0 + tx];
  __syncthreads();
  for (int i = ty; i < 64; i += 4) dst[(c0 + i) * rows + r0 + tx] = tile[tx][i];
}

__global__ void or_status_kernel(const int32_t* __restrict__ src, int32_t* __restrict__ dst) {
  if (threadIdx.x == 0 && *src) set_flag(dst, *src);
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace lora

namespace lora_host {
using namespace lora;

static unsigned grid_for(int64_t work, int per_block, int cap = 4096) {
  int64_t b = cdiv(work, per_block);
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (unsigned)b;
}

lora_status launch_logprob_merge(const float* part_m, const float* part_s, const float* zt,
                                 const int32_t* targets, int64_t n, int tiles, int64_t vocab,
                                 float* logprobs, float* lse, int32_t* status, hipStream_t s) {
  if (n <= 0) return LORA_OK;
  hipLaunchKernelGGL(logprob_merge_kernel, dim3((unsigned)cdiv(n, 64)), dim3(64 * MERGE_WAVES), 0,
                     s, part_m, part_s, zt, targets, n, tiles, vocab, logprobs, lse, status);
  return launch_check("logprob_merge");
}

lora_status launch_loss(int kind, int64_t n, const float* logp, const float* w, const float* adv,
                        const float* samp, const float* g, float clip_lo, float clip_hi,
                        double* partial, float* loss_out, float* dlogp, int32_t* status,
                        hipStream_t s) {
  const int64_t nb = cdiv(n, LOSS_ROWS);
  if (nb > 0) {
    hipLaunchKernelGGL(loss_rows_kernel, dim3((unsigned)nb), dim3(256), 0, s, kind, n, logp, w,
                       adv, samp, g, clip_lo, clip_hi, partial, dlogp, status);
    lora_status st = launch_check("loss_rows");
    if (st) return st;
  }
  hipLaunchKernelGGL(loss_sum_kernel, dim3(1), dim3(256), 0, s, partial, (int)nb, loss_out);
  return launch_check("loss_sum");
}

lora_status launch_adam_multi(int n_seg, const int64_t* off, const int64_t* cnt,
                              const float* step_size, const float* inv_sqrt_bc2, float* p,
                              const float* g, float* m, float* v, float lr, float beta1,
                              float beta2, float eps, float wd, uint16_t* p_bf16, int32_t* skip,
                              int32_t* status, hipStream_t s) {
  lora_status st = launch_fill_i32(skip, n_seg, 0, s);
  if (st) return st;
  std::vector<AdamSegs> launches;
  std::vector<int32_t> blocks_of;
  for (int s0 = 0; s0 < n_seg; s0 += ADAM_SEGS) {
    AdamSegs sg{};
    sg.n = std::min(ADAM_SEGS, n_seg - s0);
    sg.seg0 = s0;
    int32_t blocks = 0;
    for (int i = 0; i < sg.n; ++i) {
      sg.off[i] = off[s0 + i];
      sg.cnt[i] = cnt[s0 + i];
      sg.step_size[i] = step_size[s0 + i];
      sg.inv_sqrt_bc2[i] = inv_sqrt_bc2[s0 + i];
      sg.blk0[i] = blocks;
      blocks += (int32_t)cdiv(cnt[s0 + i], ADAM_BLOCK_ELEMS);
    }
    sg.blk0[sg.n] = blocks;
    if (blocks == 0) continue;
    launches.push_back(sg);
    blocks_of.push_back(blocks);
  }
  for (size_t i = 0; i < launches.size(); ++i) {
    hipLaunchKernelGGL(adam_check_kernel, dim3(blocks_of[i]), dim3(256), 0, s, launches[i], g, skip,
                       status);
    st = launch_check("adam_check");
    if (st) return st;
  }
  for (size_t i = 0; i < launches.size(); ++i) {
    hipLaunchKernelGGL(adam_multi_kernel, dim3(blocks_of[i]), dim3(256), 0, s, launches[i], p, g, m,
                       v, lr, beta1, beta2, eps, wd, p_bf16, skip);
    st = launch_check("adam_multi");
    if (st) return st;
  }
  return LORA_OK;
}

lora_status launch_swiglu_fwd(int64_t n, const uint16_t* g, const uint16_t* u, uint16_t* h,
                              hipStream_t s) {
  if (n <= 0) return LORA_OK;
  hipLaunchKernelGGL(swiglu_kernel<false>, dim3(grid_for(cdiv(n, 8), 256)), dim3(256), 0, s, n,
                     (const uint16_t*)nullptr, g, u, h, (uint16_t*)nullptr);
  return launch_check("swiglu_fwd");
}

lora_status launch_swiglu_bwd(int64_t n, const uint16_t* dh, const uint16_t* g,
                              const uint16_t* u, uint16_t* dg, uint16_t* du, hipStream_t s) {
  if (n <= 0) return LORA_OK;
  hipLaunchKernelGGL(swiglu_kernel<true>, dim3(grid_for(cdiv(n, 8), 256)), dim3(256), 0, s, n, dh,
                     g, u, dg, du);
  return launch_check("swiglu_bwd");
}

// out = bf16(a + b), the sum taken in fp32 (one rounding); 8 elements per step.
__global__ __launch_bounds__(256) void add_bf16_kernel(int64_t n, const uint16_t* __restrict__ a,
                                                       const uint16_t* __restrict__ b,
                                                       uint16_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n8 = n / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const uint4 x = ((const uint4*)a)[i], y = ((const uint4*)b)[i];
    const uint32_t wx[4] = {x.x, x.y, x.z, x.w}, wy[4] = {y.x, y.y, y.z, y.w};
    uint32_t r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      r[q] = pack2bf(bf2f_lo(wx[q]) + bf2f_lo(wy[q]), bf2f_hi(wx[q]) + bf2f_hi(wy[q]));
    ((uint4*)out)[i] = make_uint4(r[0], r[1], r[2], r[3]);
  }
  for (int64_t e = n8 * 8 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride)
    out[e] = f2bf(bf2f(a[e]) + bf2f(b[e]));
}

lora_status launch_add_bf16(int64_t n, const uint16_t* a, const uint16_t* b, uint16_t* out,
                            hipStream_t s) {
  if (n <= 0) return LORA_OK;
  hipLaunchKernelGGL(add_bf16_kernel, dim3(grid_for(cdiv(n, 8), 256)), dim3(256), 0, s, n, a, b,
                     out);
  return launch_check("add_bf16");
}

lora_status launch_transpose_bf16(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t cols,
                                  hipStream_t s) {
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)(cols / 64), (unsigned)(rows / 64)),
                     dim3(256), 0, s, src, dst, rows, cols);
  return launch_check("transpose_bf16");
}

lora_status launch_or_status(const int32_t* src, int32_t* dst, hipStream_t s) {
  hipLaunchKernelGGL(or_status_kernel, dim3(1), dim3(64), 0, s, src, dst);
  return launch_check("or_status");
}

lora_status launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(n, 256, 1024)), dim3(256), 0, s, p, n, v);
  return launch_check("fill_i32");
}

}  // namespace lora_host
