// Segmented LoRA kernels for gfx950 (SGMV-style: tinker-ticks, "How the SGMV
// kernel works" -- one launch per phase serves every adapter in the batch).
//
// Rows are visited in segment order: position p of the stable order `perm`
// holds token perm[p]; adapter a owns positions offsets[a]..offsets[a+1].
// Each launch's blocks are cut per adapter (tile prefix sums from the segment
// builder), so a block only ever touches one adapter's factors.  Per-token
// vectors (u, v) and the big row-major operands stay in token order; the
// kernels gather rows through perm.
//
//   shrink   out[t][c] = sum_k in[t][k] M_a[c][k]      (u = A_a x, v = B_a^T g)
//            16 rows per block, the four waves split K, one LDS reduction.
//   (the expand y += s B_a u / dx += s A_a^T v runs inside the base GEMM's
//    epilogue: gemm.hip, lora_slab)
//   grad     T[c][j] = s_a sum_{t in chunk} P[t][c] Q[t][j]  (dB_a, dA_a)
//            one block per (token chunk of an adapter, 256 columns); Q rows are
//            register-transposed into LDS so both MFMA operands are
//            K(=token)-contiguous; P (fp32) is split hi+lo.  Adapters with one
//            chunk write the result directly, others write chunk partials that
//            `grad_finalize` sums in chunk order (deterministic, no atomics).
#include "common.hpp"
#include "sgmv.hpp"

namespace lora {

// Swizzled index of a 16-byte chunk in an LDS tile whose rows hold 8 chunks.
__device__ __forceinline__ int sw8(int row, int chunk) { return row * 8 + (chunk ^ lds_sw(row)); }

struct TileInfo {
  int a;
  int p0;     // first position (segment order)
  int rows;   // rows in this tile
};

__device__ __forceinline__ bool tile_of(const int32_t* pre, const int32_t* offsets, int n_ad,
                                        int tile, int tm, TileInfo& ti) {
  if (tile >= pre[n_ad]) return false;
  const int a = find_bucket(pre, n_ad + 1, tile);
  ti.a = a;
  ti.p0 = offsets[a] + (tile - pre[a]) * tm;
  ti.rows = min(tm, offsets[a + 1] - ti.p0);
  return true;
}

// ------------------------------------------------------------------ shrink
template <int NB>
__device__ __forceinline__ void shrink_body(const uint16_t* __restrict__ in, int64_t ld_in, int K,
                                            const uint16_t* __restrict__ mat, int r, int tok,
                                            int lane, int wave, f32x4* acc) {
  const int KB = K / 32;
  const int kb0 = wave * KB / 4, kb1 = (wave + 1) * KB / 4;
  const int ko = 8 * (lane >> 4);
  const int c = lane & 15;
  const uint16_t* xrow = in + (int64_t)(tok >= 0 ? tok : 0) * ld_in + ko;
  const uint16_t* mrow[NB];
  bool mok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    mok[nb] = (nb * 16 + c) < r;
    mrow[nb] = mat + (int64_t)(mok[nb] ? nb * 16 + c : 0) * K + ko;
  }
  const uint4 z = make_uint4(0, 0, 0, 0);
  int kb = kb0;
  for (; kb + 4 <= kb1; kb += 4) {
    uint4 xv[4], mv[4][NB];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      xv[u] = tok >= 0 ? *(const uint4*)(xrow + (kb + u) * 32) : z;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) mv[u][nb] = mok[nb] ? *(const uint4*)(mrow[nb] + (kb + u) * 32) : z;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma16(as_bf16x8(xv[u]), as_bf16x8(mv[u][nb]), acc[nb]);
  }
  for (; kb < kb1; ++kb) {
    uint4 xv = tok >= 0 ? *(const uint4*)(xrow + kb * 32) : z;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint4 mv = mok[nb] ? *(const uint4*)(mrow[nb] + kb * 32) : z;
      acc[nb] = mfma16(as_bf16x8(xv), as_bf16x8(mv), acc[nb]);
    }
  }
}

// grid.x = tile bound; grid.y = 2: y == 0 computes tiles, y == 1 zeroes the
// rows of tokens that belong to no active adapter (positions >= offsets[n_ad]
// or inside an inactive adapter's segment).
__global__ __launch_bounds__(256) void shrink_kernel(
    const uint16_t* __restrict__ in, int64_t ld_in, int K, const uint16_t* __restrict__ mat_pack,
    int use_b_off, const lora_adapter_desc* __restrict__ desc, const uint8_t* __restrict__ active,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ pre16, int n_ad, int64_t n_tokens, float* __restrict__ out,
    int r_max) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.y == 1) {
    const int64_t p = (int64_t)blockIdx.x * 256 + tid;
    if (p >= n_tokens) return;
    bool dead = p >= offsets[n_ad];
    if (!dead) dead = !active[find_bucket(offsets, n_ad + 1, (int32_t)p)];
    if (dead) {
      float* o = out + (int64_t)perm[p] * r_max;
      for (int c = 0; c < r_max; ++c) o[c] = 0.f;
    }
    return;
  }
  TileInfo ti;
  if (!tile_of(pre16, offsets, n_ad, blockIdx.x, 16, ti)) return;
  const lora_adapter_desc d = desc[ti.a];
  const int r = d.rank;
  const uint16_t* mat = mat_pack + (use_b_off ? d.b_off : d.a_off);
  const int row = lane & 15;
  const int tok = row < ti.rows ? perm[ti.p0 + row] : -1;

  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nb = (r + 15) / 16;
  if (nb == 1) shrink_body<1>(in, ld_in, K, mat, r, tok, lane, wave, acc);
  else if (nb == 2) shrink_body<2>(in, ld_in, K, mat, r, tok, lane, wave, acc);
  else if (nb == 3) shrink_body<3>(in, ld_in, K, mat, r, tok, lane, wave, acc);
  else shrink_body<4>(in, ld_in, K, mat, r, tok, lane, wave, acc);

  // cross-wave reduction in a fixed order.  acc[nb][i] = D[4*(lane/16)+i][nb*16 + lane%16]
  __shared__ float red[4][16][64];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * (lane >> 4) + i][b * 16 + (lane & 15)] = acc[b][i];
  __syncthreads();
  const int orow = tid >> 4, cg = (tid & 15) * 4;
  if (orow < ti.rows && cg < r_max) {
    const int t = perm[ti.p0 + orow];
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = cg + q;
      float s = red[0][orow][c] + red[1][orow][c];
      s += red[2][orow][c];
      s += red[3][orow][c];
      v[q] = c < r ? s : 0.f;
    }
    float* o = out + (int64_t)t * r_max + cg;
    // r_max is a multiple of 8, so the 4-float group is either inside or outside
    *(float4*)o = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// ------------------------------------------------------------------ grad
constexpr int GR_TC = 1024;   // tokens per chunk (per-adapter split for balance)
constexpr int GR_TT = 64;     // tokens staged per step
constexpr int GR_NJ = 256;    // output columns per block

// mode 0 (dB): out layout [D][r] (c fastest): MFMA M = c, N = j.
// mode 1 (dA): out layout [r][D] (j fastest): MFMA M = j, N = c.
template <int NCB, int MODE>
__device__ __forceinline__ void grad_mma(const uint4* Qt, const uint4* Ph, const uint4* Pl,
                                         int lane, int wave, f32x4 (&acc)[4][4]) {
#pragma unroll
  for (int kb = 0; kb < GR_TT / 32; ++kb) {
    const int ch = kb * 4 + (lane >> 4);
    bf16x8 q[4], ph[NCB], pl[NCB];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int j = wave * 64 + jt * 16 + (lane & 15);
      q[jt] = as_bf16x8(Qt[sw8(j, ch)]);
    }
#pragma unroll
    for (int ct = 0; ct < NCB; ++ct) {
      const int c = ct * 16 + (lane & 15);
      ph[ct] = as_bf16x8(Ph[sw8(c, ch)]);
      pl[ct] = as_bf16x8(Pl[sw8(c, ch)]);
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int ct = 0; ct < NCB; ++ct) {
        if (MODE == 0) {
          acc[jt][ct] = mfma16(ph[ct], q[jt], acc[jt][ct]);
          acc[jt][ct] = mfma16(pl[ct], q[jt], acc[jt][ct]);
        } else {
          acc[jt][ct] = mfma16(q[jt], ph[ct], acc[jt][ct]);
          acc[jt][ct] = mfma16(q[jt], pl[ct], acc[jt][ct]);
        }
      }
  }
}

// grid = (chunk-slot bound, ceil(D / 256)).
template <int MODE>
__global__ __launch_bounds__(256) void grad_kernel(
    const float* __restrict__ P, int r_max, const uint16_t* __restrict__ Q, int64_t ld_q, int D,
    const lora_adapter_desc* __restrict__ desc, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ chunk_pre, int n_ad,
    float* __restrict__ out_pack, float* __restrict__ partial, int accumulate) {
  const int slot = blockIdx.x;
  TileInfo ti;
  if (!tile_of(chunk_pre, offsets, n_ad, slot, GR_TC, ti)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const lora_adapter_desc d = desc[ti.a];
  const int r = d.rank;
  const int j0 = blockIdx.y * GR_NJ;
  const int nchunks = chunk_pre[ti.a + 1] - chunk_pre[ti.a];

  __shared__ uint4 Qt[GR_NJ * 8];   // [256 j][64 t] bf16, swizzled
  __shared__ uint4 Ph[64 * 8];      // [64 c][64 t]
  __shared__ uint4 Pl[64 * 8];
  uint16_t* Ph16 = (uint16_t*)Ph;
  uint16_t* Pl16 = (uint16_t*)Pl;

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int jc = tid & 31;        // 8-column group of Q
  const int toct = tid >> 5;      // 8-token group
  const int pt = tid >> 2;        // P staging: token
  const int pcg = (tid & 3) * 16; // P staging: first of 16 columns
  const int ncb = (r + 15) / 16;

  for (int t0 = 0; t0 < ti.rows; t0 += GR_TT) {
    // ---- stage Q^T: 8 tokens x 8 columns per thread, transposed in registers
    uint32_t w[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tr = t0 + toct * 8 + i;
      const int j = j0 + jc * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tr < ti.rows && j < D) v = *(const uint4*)(Q + (int64_t)perm[ti.p0 + tr] * ld_q + j);
      w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
    }
#pragma unroll
    for (int qc = 0; qc < 8; ++qc) {
      const int wd = qc >> 1, sh = (qc & 1) * 16;
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = (w[2 * k][wd] >> sh) & 0xFFFFu;
        const uint32_t hi = (w[2 * k + 1][wd] >> sh) & 0xFFFFu;
        o[k] = lo | (hi << 16);
      }
      Qt[sw8(jc * 8 + qc, toct)] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    // ---- stage P^T as hi/lo bf16: token pt, columns pcg..pcg+15
    {
      const int tr = t0 + pt;
      const bool ok = tr < ti.rows;
      const float* pp = P + (int64_t)(ok ? perm[ti.p0 + tr] : 0) * r_max;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int c = pcg + q;
        float f = (ok && c < r) ? pp[c] : 0.f;
        uint16_t h, l;
        split_bf16(f, h, l);
        const int idx = c * 64 + (((pt >> 3) ^ lds_sw(c)) << 3) + (pt & 7);
        Ph16[idx] = h;
        Pl16[idx] = l;
      }
    }
    __syncthreads();
    if (ncb == 1) grad_mma<1, MODE>(Qt, Ph, Pl, lane, wave, acc);
    else if (ncb == 2) grad_mma<2, MODE>(Qt, Ph, Pl, lane, wave, acc);
    else if (ncb == 3) grad_mma<3, MODE>(Qt, Ph, Pl, lane, wave, acc);
    else grad_mma<4, MODE>(Qt, Ph, Pl, lane, wave, acc);
    __syncthreads();
  }

  // ---- write.  Region of this adapter: D*r floats.
  const int64_t base = MODE == 0 ? d.b_off : d.a_off;
  const bool direct = nchunks == 1;
  float* dst = direct ? out_pack + base : partial + (int64_t)slot * D * r_max;
  const float s = d.scale;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      if (ct >= ncb) continue;
      if (MODE == 0) {
        // D[c][j]: lane holds c = ct*16 + 4*(lane/16) + i, j = jt*16 + lane%16
        const int c = ct * 16 + 4 * (lane >> 4);
        const int j = j0 + wave * 64 + jt * 16 + (lane & 15);
        if (c >= r || j >= D) continue;
        float4* p = (float4*)(dst + (int64_t)j * r + c);
        float4 v = make_float4(s * acc[jt][ct][0], s * acc[jt][ct][1], s * acc[jt][ct][2], s * acc[jt][ct][3]);
        if (direct && accumulate) {
          float4 o = *p;
          v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
        }
        *p = v;
      } else {
        // D[j][c]: lane holds j = jt*16 + 4*(lane/16) + i, c = ct*16 + lane%16
        const int j = j0 + wave * 64 + jt * 16 + 4 * (lane >> 4);
        const int c = ct * 16 + (lane & 15);
        if (c >= r || j >= D) continue;
        float4* p = (float4*)(dst + (int64_t)c * D + j);
        float4 v = make_float4(s * acc[jt][ct][0], s * acc[jt][ct][1], s * acc[jt][ct][2], s * acc[jt][ct][3]);
        if (direct && accumulate) {
          float4 o = *p;
          v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
        }
        *p = v;
      }
    }
}

// grid = (n_ad, blocks over D*r_max/1024).  Sums the chunk partials of
// adapters with several chunks, in chunk order; with accumulate == 0 writes
// zeros for active adapters that own no token.
__global__ __launch_bounds__(256) void grad_finalize_kernel(
    const lora_adapter_desc* __restrict__ desc, const uint8_t* __restrict__ active,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ chunk_pre, int D,
    int r_max, int mode, float* __restrict__ out_pack, const float* __restrict__ partial,
    int accumulate) {
  const int a = blockIdx.x;
  if (!active[a]) return;
  const int count = offsets[a + 1] - offsets[a];
  const int s0 = chunk_pre[a], ns = chunk_pre[a + 1] - s0;
  const bool zero = count == 0 && !accumulate;
  if (!zero && ns < 2) return;
  const lora_adapter_desc d = desc[a];
  const int64_t n = (int64_t)D * d.rank;
  float* dst = out_pack + (mode == 0 ? d.b_off : d.a_off);
  for (int64_t e = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4; e < n;
       e += (int64_t)gridDim.y * 256 * 4) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!zero) {
      for (int q = 0; q < ns; ++q) {
        const float4 p = *(const float4*)(partial + (int64_t)(s0 + q) * D * r_max + e);
        v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
      }
      if (accumulate) {
        const float4 o = *(const float4*)(dst + e);
        v.x = o.x + v.x; v.y = o.y + v.y; v.z = o.z + v.z; v.w = o.w + v.w;
      }
    }
    *(float4*)(dst + e) = v;
  }
}

// ------------------------------------------------------------------ adapter transposes
// AT[a_off + k*r + c] = A[a_off + c*d_in + k]  (A_a^T, [d_in][r])
// BT[b_off + c*d_out + j] = B[b_off + j*r + c]  (B_a^T, [r][d_out])
__global__ __launch_bounds__(256) void adapter_transpose_kernel(
    const uint16_t* __restrict__ A_pack, const uint16_t* __restrict__ B_pack,
    const lora_adapter_desc* __restrict__ desc, const uint8_t* __restrict__ active, int64_t d_in,
    int64_t d_out, uint16_t* __restrict__ AT, uint16_t* __restrict__ BT) {
  const int a = blockIdx.x;
  if (!active[a]) return;
  const lora_adapter_desc d = desc[a];
  const int r = d.rank;
  const int groups = r / 8;
  // A^T: one thread per (k, group of 8 c): 8 strided reads, one 16-byte write
  for (int64_t e = (int64_t)blockIdx.y * 256 + threadIdx.x; e < d_in * groups;
       e += (int64_t)gridDim.y * 256) {
    const int64_t k = e / groups;
    const int g = (int)(e % groups);
    uint16_t v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = A_pack[d.a_off + (int64_t)(g * 8 + q) * d_in + k];
    *(uint4*)(AT + d.a_off + k * r + g * 8) =
        make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
  }
  // B^T: one thread per j: one 16-byte read per group, r scattered 2-byte writes
  for (int64_t j = (int64_t)blockIdx.y * 256 + threadIdx.x; j < d_out; j += (int64_t)gridDim.y * 256) {
    for (int g = 0; g < groups; ++g) {
      const uint4 v = *(const uint4*)(B_pack + d.b_off + j * r + g * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 8; ++q)
        BT[d.b_off + (int64_t)(g * 8 + q) * d_out + j] = (uint16_t)(w[q >> 1] >> ((q & 1) * 16));
    }
  }
}

}  // namespace lora

namespace lora_host {
using namespace lora;

lora_status launch_shrink(const uint16_t* in, int64_t ld_in, int K, const uint16_t* mat_pack,
                          int use_b_off, const lora_adapter_desc* desc, const uint8_t* active,
                          const int32_t* perm, const int32_t* offsets, const int32_t* pre16,
                          int n_ad, int64_t n_tokens, float* out, int r_max, hipStream_t s) {
  if (n_tokens <= 0) return LORA_OK;
  const int64_t bound = cdiv(n_tokens, 16) + n_ad;
  hipLaunchKernelGGL(shrink_kernel, dim3((unsigned)bound, 2), dim3(256), 0, s, in, ld_in, K,
                     mat_pack, use_b_off, desc, active, perm, offsets, pre16, n_ad, n_tokens, out,
                     r_max);
  return launch_check("shrink");
}

lora_status launch_grad(int mode, const float* P, int r_max, const uint16_t* Q, int64_t ld_q,
                        int D, const lora_adapter_desc* desc, const uint8_t* active,
                        const int32_t* perm, const int32_t* offsets, const int32_t* chunk_pre,
                        int n_ad, int64_t n_tokens, float* out_pack, float* partial,
                        int accumulate, hipStream_t s) {
  if (n_tokens > 0) {
    const int64_t bound = cdiv(n_tokens, GR_TC) + n_ad;
    dim3 grid((unsigned)bound, (unsigned)cdiv(D, GR_NJ));
    if (mode == 0)
      hipLaunchKernelGGL(grad_kernel<0>, grid, dim3(256), 0, s, P, r_max, Q, ld_q, D, desc, perm,
                         offsets, chunk_pre, n_ad, out_pack, partial, accumulate);
    else
      hipLaunchKernelGGL(grad_kernel<1>, grid, dim3(256), 0, s, P, r_max, Q, ld_q, D, desc, perm,
                         offsets, chunk_pre, n_ad, out_pack, partial, accumulate);
    lora_status st = launch_check("grad");
    if (st) return st;
  }
  const int64_t per = (int64_t)D * r_max;
  const unsigned gy = (unsigned)std::max<int64_t>(1, std::min<int64_t>(64, cdiv(per, 1024)));
  hipLaunchKernelGGL(grad_finalize_kernel, dim3(n_ad, gy), dim3(256), 0, s, desc, active, offsets,
                     chunk_pre, D, r_max, mode, out_pack, partial, accumulate);
  return launch_check("grad_finalize");
}

int64_t grad_partial_floats(int64_t n_tokens, int n_ad, int64_t D, int r_max) {
  return (cdiv(n_tokens, GR_TC) + n_ad) * D * r_max;
}

lora_status launch_adapter_transpose(const uint16_t* A_pack, const uint16_t* B_pack,
                                     const lora_adapter_desc* desc, const uint8_t* active,
                                     int n_ad, int64_t d_in, int64_t d_out, uint16_t* AT,
                                     uint16_t* BT, hipStream_t s) {
  const unsigned gy = (unsigned)std::max<int64_t>(1, std::min<int64_t>(64, cdiv(std::max(d_in * 8, d_out), 256)));
  hipLaunchKernelGGL(adapter_transpose_kernel, dim3(n_ad, gy), dim3(256), 0, s, A_pack, B_pack,
                     desc, active, d_in, d_out, AT, BT);
  return launch_check("adapter_transpose");
}

}  // namespace lora_host
