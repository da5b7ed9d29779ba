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
//            32 rows per block streamed through an LDS-DMA ring (128 rows for
//            large batches, same per-row summation order).
//   (the expand y += s B_a u / dx += s A_a^T v runs inside the base GEMM's
//    epilogue: gemm.hip, lora_expand; few-row batches: gemm_fewrow_kernel)
//   grad     T[c][j] = s_a sum_{t in chunk} P[t][c] Q[t][j]  (dB_a, dA_a)
//            one block per (token chunk of an adapter, 256 columns); Q and P
//            stream through an LDS-DMA ring and Q is transposed on the LDS
//            read (ds_read_b64_tr_b16) so both MFMA operands are
//            K(=token)-contiguous; P (fp32) is split hi+lo.  Adapters with one
//            chunk write the result directly, others write chunk partials that
//            `grad_finalize` sums in chunk order (deterministic, no atomics).
#include <type_traits>

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

// WAVE: the bucket search by a whole wave's ballots (fewer dependent loads;
// the shrink's lookup sits on its critical path), else the binary search
// (fewer registers; the gradient items measured no faster with the wave one).
template <bool WAVE = true>
__device__ __forceinline__ bool tile_of(const int32_t* pre, const int32_t* offsets, int n_ad,
                                        int tile, int tm, TileInfo& ti) {
  if (tile >= pre[n_ad]) return false;
  const int a = WAVE ? find_bucket_wave(pre, n_ad + 1, tile) : find_bucket(pre, n_ad + 1, tile);
  ti.a = a;
  ti.p0 = offsets[a] + (tile - pre[a]) * tm;
  ti.rows = min(tm, offsets[a + 1] - ti.p0);
  return true;
}

// Work items [0, total) of a one-block-per-CU grid, handed out so that each
// XCD walks a contiguous item range (the dispatcher places block b on XCD
// b % 8; items of one XCD then read one contiguous stretch of memory, which
// the memory system serves markedly faster than an interleaved one).
// gridDim.x must be a multiple of 8.
struct ItemRange {
  int first, step, end;
};
__device__ __forceinline__ ItemRange xcd_items(int total) {
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int base = total >> 3, rem = total & 7;
  const int start = xcd * base + min(xcd, rem);
  return ItemRange{start + loc, (int)(gridDim.x >> 3), start + base + (xcd < rem ? 1 : 0)};
}

// ------------------------------------------------------------------ shrink
// out[t][c] = sum_k in[t][k] M_a[c][k] for the 32 rows of one adapter tile.
// Rows (gathered through perm) and the factor M_a stream through a 5-stage
// LDS ring of k = 128 slices by LDS-DMA (issued from inline assembly, four
// stages ahead, explicit vmcnt waits; the compiler cannot track which stage a
// DMA writes).  Each LDS row of the token tile is 256 B = 16 chunks, chunk c
// stored at c ^ (row & 15), so the fragment reads of 16 consecutive rows are
// conflict-free.  Waves 0, 1 take rows 0..15, 16..31 over the even 32-k
// blocks of every stage, waves 2, 3 the same rows over the odd blocks; the
// two chains of a row meet once per 1024-k chunk (the summation order below).
// The factor is either A_a (KM = false: [r][K], one LDS row per rank, stored
// like the token rows) or B_a read in place for M_a = B_a^T (KM = true:
// B_a is [K][r], so a k slice is one contiguous block of 128 x r values; it
// is copied flat and the MFMA operand, 8 consecutive k of one rank, comes
// from two transposing reads ds_read_b64_tr_b16).
constexpr int SH_TM = 32;
constexpr int SH_KC = 128;
// Ring depth (deeper rings measured no faster).
template <int NB>
constexpr int sh_nst() {
  return 5;
}
constexpr int SH_XSLOTS = SH_TM * 16;          // uint4 slots of the row tile per stage

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

__device__ __forceinline__ void dma16(const void* g, uint32_t m0v) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0v), "v"(g) : "memory");
}

template <int VM>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(VM) : "memory");
}

// Row maps of a shrink: position p reads input row in[p] and writes output
// row out[p] (identity when null); rowscale[p] (nullable) multiplies s_a.
struct ShrinkRows {
  const int32_t* in;
  const int32_t* out;
  const float* rowscale;
};

// Second factor of a dual shrink (same input rows, another adapter table, KM
// = false only): tile ranks [c2, c2 + r) come from mat and go to out.
struct ShrinkSecond {
  const uint16_t* mat;   // null: single shrink
  int r, c2;
  float scale;
  uint16_t* out;
};

// Summation order of every shrink, whatever its tile height or K split: k
// falls into chunks of SHRINK_KCH; within a chunk the 32-k blocks of even and
// of odd parity each form one MFMA chain in increasing k, and the chunk's sum
// is S_c = even + odd; the row's value is T = (((0 + S_0) + S_1) + ...) in
// chunk order, scaled by s_a (rounded to fp32) and then split into the hi/lo
// planes.  So a row's u has the same bits in the 32-row and 128-row tiles and
// in a launch that splits K over blocks (the chunk sums then go through
// `part` to shrink_fold_kernel, which folds them in the same order).
constexpr int SHRINK_KCH = 1024;

// Scale and split tile ranks [c0, c0 + rr) of the rows of one tile into the
// planes of dst; val(row, c) is the row's folded sum T for rank c0 + c.
template <class V>
__device__ __forceinline__ void shrink_emit(V&& val, uint16_t* __restrict__ dst, int c0, int rr,
                                            float sc, const ShrinkRows& rm, int p0, int rows,
                                            int tm, int64_t plane, int r_max) {
  // the scaled value is rounded to fp32 before the hi/lo split (no product
  // fused into the residual), in every tile height alike
#pragma clang fp contract(off)
  for (int e = threadIdx.x; e < tm * (r_max / 4); e += blockDim.x) {
    const int row = e / (r_max / 4), cg = (e % (r_max / 4)) * 4;
    if (row >= rows) continue;
    const int prow = p0 + row;
    const float sc_row = rm.rowscale ? sc * rm.rowscale[prow] : sc;
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = cg + q;
      v[q] = c < rr ? sc_row * val(row, c0 + c) : 0.f;
    }
    uint32_t h01, l01, h23, l23;
    split2_bf16(v[0], v[1], h01, l01);
    split2_bf16(v[2], v[3], h23, l23);
    uint16_t* o = dst + (int64_t)(rm.out ? rm.out[prow] : prow) * r_max + cg;
    *(uint2*)o = make_uint2(h01, h23);
    *(uint2*)(o + plane) = make_uint2(l01, l23);
  }
}

// Chunks [c0, c1) of one 32-row tile.  part == nullptr: every chunk of K, the
// sums folded here and written as planes.  Otherwise the chunk sums S_c go to
// part[c][row][64] (fp32) and nothing else is written.
template <int NB, bool KM>
__device__ __forceinline__ void shrink_tile(const uint16_t* __restrict__ in, int64_t ld_in, int K,
                                            const uint16_t* __restrict__ mat, int r, float scale,
                                            const ShrinkSecond sec, const ShrinkRows rm, int p0,
                                            int rows, uint4* lds, uint16_t* __restrict__ out,
                                            int64_t plane, int r_max, int c0, int c1,
                                            float* __restrict__ part) {
  constexpr int MSLOTS = NB * 16 * 16;                 // factor tile slots per stage
  constexpr int STAGE = SH_XSLOTS + MSLOTS;
  constexpr int PER_WAVE = 2 + NB;                     // DMA instructions per wave per stage
  constexpr int NST = sh_nst<NB>();
  constexpr int CST = SHRINK_KCH / SH_KC;              // stages per chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int KT = (K + SH_KC - 1) / SH_KC;
  const int kt0 = c0 * CST, kt1 = min(KT, c1 * CST);   // this call's stages

  // DMA sources of this lane: 2 row-tile instructions, NB factor instructions
  const uint16_t* xsrc[2];
  int xchunk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (wave * 2 + i) * 4 + (lane >> 4);
    const int pr = p0 + (row < rows ? row : 0);
    const int t = rm.in ? rm.in[pr] : pr;
    xchunk[i] = (lane & 15) ^ (row & 15);
    xsrc[i] = in + (int64_t)t * ld_in;
  }
  // factor sources: KM = false, rank row c, chunk mchunk; KM = true, flat
  // element offset of this lane's 16 bytes within a k slice (128 rows of r)
  const uint16_t* msrc[NB];
  int mchunk[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if constexpr (KM) {
      msrc[i] = mat;
      mchunk[i] = ((wave * NB + i) * 64 + lane) * 8;
    } else {
      const int c = (wave * NB + i) * 4 + (lane >> 4);
      mchunk[i] = (lane & 15) ^ (c & 15);
      if (sec.mat && c >= sec.c2) {
        const int c2 = c - sec.c2;
        msrc[i] = sec.mat + (int64_t)(c2 < sec.r ? c2 : sec.r - 1) * K;
      } else {
        msrc[i] = mat + (int64_t)(c < r ? c : r - 1) * K;
      }
    }
  }
  const int64_t m_last = (int64_t)K * r - 8;   // KM: last 16-byte source of the factor
  auto issue = [&](int st, int kt) {
    const int k0 = kt * SH_KC;
    uint4* base = lds + st * STAGE;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = min(k0 + xchunk[i] * 8, K - 8);
      dma16(xsrc[i] + k, __builtin_amdgcn_readfirstlane(lds_u32(base + (wave * 2 + i) * 64)));
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const uint32_t dst =
          __builtin_amdgcn_readfirstlane(lds_u32(base + SH_XSLOTS + (wave * NB + i) * 64));
      if constexpr (KM) {
        // past the factor's last row: clamped; those values only meet k >= K,
        // which no wave multiplies
        dma16(msrc[i] + min((int64_t)k0 * r + mchunk[i], m_last), dst);
      } else {
        const int k = min(k0 + mchunk[i] * 8, K - 8);
        dma16(msrc[i] + k, dst);
      }
    }
  };

#pragma unroll
  for (int st = 0; st < NST - 1; ++st) issue(st, min(kt0 + st, kt1 - 1));
  wait_vm_barrier<(NST - 2) * PER_WAVE>();

  // wave w: rows 16 (w & 1) .. + 15, and the 32-k blocks of parity w >> 1
  // (blocks kp and kp + 2 of each 128-k stage): each row has an even-block and
  // an odd-block chain per chunk.  Between chunks the odd waves hand their
  // chains to the even waves through LDS (fo), which add them (S_c) and fold
  // S_c into tot, or store it to part.
  f32x4 acc[NB], tot[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = tot[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15;
  const int rh = wave & 1, kp = wave >> 1;
  float* fo = (float*)(lds + NST * STAGE);   // [SH_TM][64], past the ring

  int kt = kt0;
  for (int c = c0; c < c1; ++c) {
    const int kte = min(kt1, (c + 1) * CST);
    for (; kt < kte; ++kt) {
      const int st = (kt - kt0) % NST;
      issue((kt - kt0 + NST - 1) % NST, min(kt + NST - 1, kt1 - 1));
      const uint4* xt = lds + st * STAGE;
      const uint4* mt = xt + SH_XSLOTS;
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        const int bb = kp + 2 * bi;              // 32-k block of the stage
        if (kt * SH_KC + bb * 32 >= K) continue;
        const int ch = 4 * bb + (lane >> 4);     // logical chunk of this lane's fragments
        bf16x8 xa, mb[NB];
        {
          const int row = rh * 16 + fr;
          xa = as_bf16x8(xt[row * 16 + (ch ^ (row & 15))]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if constexpr (KM) {
            // rows k = 8 ch + {0..3} and {4..7}; in each 16-lane group, lane 4q + j
            // addresses row k0 + q, ranks 16 b + 4 j .. + 3, and receives rank
            // 16 b + (lane & 15) of the four rows
            const int q = (lane >> 2) & 3, j = lane & 3;
            const uint32_t off = (uint32_t)(((8 * ch + q) * r + 16 * b + 4 * j) * 2);
            const uint2 lo = tr_read(mt, off);
            const uint2 hi = tr_read(mt, off + (uint32_t)(4 * r * 2));
            mb[b] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
          } else {
            const int cc = b * 16 + fr;
            mb[b] = as_bf16x8(mt[cc * 16 + (ch ^ (cc & 15))]);
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = mfma16(xa, mb[b], acc[b]);
      }
      wait_vm_barrier<(NST - 2) * PER_WAVE>();
    }
    // chunk c's end.  acc[b][i] = chain of D[16 rh + 4 (lane / 16) + i][16 b + lane % 16]
    if (kp == 1) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          fo[(rh * 16 + 4 * (lane >> 4) + i) * 64 + b * 16 + (lane & 15)] = acc[b][i];
    }
    __syncthreads();
    if (kp == 0) {
      float* pc = part ? part + (size_t)c * (SH_TM * 64) : nullptr;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int idx = (rh * 16 + 4 * (lane >> 4) + i) * 64 + b * 16 + (lane & 15);
          const float sc_sum = acc[b][i] + fo[idx];
          if (pc) pc[idx] = sc_sum;
          else tot[b][i] = tot[b][i] + sc_sum;
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    // (fo is written again at the next chunk's end, after that chunk's stage
    // barriers, which the even waves reach after these reads)
  }
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  if (part) return;

  float* red = (float*)lds;  // [SH_TM][64]: the folded sums
  if (kp == 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(rh * 16 + 4 * (lane >> 4) + i) * 64 + b * 16 + (lane & 15)] = tot[b][i];
  }
  __syncthreads();
  auto val = [&](int row, int c) { return red[row * 64 + c]; };
  shrink_emit(val, out, 0, r, scale, rm, p0, rows, SH_TM, plane, r_max);
  if (!KM && sec.mat) shrink_emit(val, sec.out, sec.c2, sec.r, sec.scale, rm, p0, rows, SH_TM, plane, r_max);
}

// The same product for large batches over 128-row adapter tiles: each factor
// row then streams once per 128 rows instead of once per 32 (in the 32-row
// kernel the factor is half of each CU's traffic).  Stages of k = 64, one
// 128-byte line per row; wave w owns rows 32w .. 32w + 31 of the tile over
// every k of a stage, so the partial products need no cross-wave sum.  LDS
// rows are 128 B with 16-byte chunk c stored at c ^ ((row >> 1) & 7): the
// fragment reads of 16 consecutive rows hit distinct banks.  The factor tile of
// a stage holds FB = 2 (ranks <= 32) or 4 rank blocks of 16 (rows clamped to
// the last rank; KM: a flat copy of the k slice, clamped to the factor's end),
// so every wave issues the same DMA count.
constexpr int ST_TM = 128;
constexpr int ST_KC = 64;
constexpr int ST_NST = 5;
constexpr int ST_XSLOTS = ST_TM * 8;   // uint4 slots of the row tile per stage (16 KB)
__device__ __forceinline__ int st_sw(int row) { return (row >> 1) & 7; }
template <int NB> constexpr int st_fb() { return NB <= 2 ? 2 : 4; }

template <int NB, bool KM>
__device__ __forceinline__ void shrink_tall_tile(const uint16_t* __restrict__ in, int64_t ld_in,
                                                 int K, const uint16_t* __restrict__ mat, int r,
                                                 float scale, const ShrinkSecond sec,
                                                 const ShrinkRows rm, int p0, int rows, uint4* lds,
                                                 uint16_t* __restrict__ out, int64_t plane,
                                                 int r_max) {
  constexpr int FB = st_fb<NB>();
  constexpr int MSLOTS = FB * 16 * 8;              // factor tile slots per stage
  constexpr int STAGE = ST_XSLOTS + MSLOTS;
  constexpr int PER_WAVE = 4 + FB / 2;             // DMA instructions per wave per stage
  constexpr int NST = ST_NST;
  constexpr int CST = SHRINK_KCH / ST_KC;   // stages per chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int KT = K / ST_KC;

  // DMA sources of this lane: 4 row instructions (this wave's 32 rows, 8 per
  // instruction: lane L -> row L / 8, physical chunk L % 8), FB / 2 factor ones
  const uint16_t* xsrc[4];
  int xchunk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wave * 32 + i * 8 + (lane >> 3);
    const int pr = p0 + (row < rows ? row : 0);
    const int t = rm.in ? rm.in[pr] : pr;
    xchunk[i] = (lane & 7) ^ st_sw(row);
    xsrc[i] = in + (int64_t)t * ld_in;
  }
  const uint16_t* msrc[FB / 2];
  int mchunk[FB / 2];
#pragma unroll
  for (int i = 0; i < FB / 2; ++i) {
    const int ins = wave * (FB / 2) + i;             // factor instruction of the stage
    if constexpr (KM) {
      msrc[i] = mat;
      mchunk[i] = (ins * 64 + lane) * 8;             // element offset within the k slice
    } else {
      const int c = ins * 8 + (lane >> 3);           // rank row
      mchunk[i] = (lane & 7) ^ st_sw(c);
      if (sec.mat && c >= sec.c2) {
        const int c2 = c - sec.c2;
        msrc[i] = sec.mat + (int64_t)(c2 < sec.r ? c2 : sec.r - 1) * K;
      } else {
        msrc[i] = mat + (int64_t)(c < r ? c : r - 1) * K;
      }
    }
  }
  const int64_t m_last = (int64_t)K * r - 8;   // KM: last 16-byte source of the factor
  auto issue = [&](int st, int kt) {
    const int k0 = kt * ST_KC;
    uint4* base = lds + st * STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16(xsrc[i] + k0 + xchunk[i] * 8,
            __builtin_amdgcn_readfirstlane(lds_u32(base + (wave * 4 + i) * 64)));
#pragma unroll
    for (int i = 0; i < FB / 2; ++i) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          lds_u32(base + ST_XSLOTS + (wave * (FB / 2) + i) * 64));
      if constexpr (KM)
        dma16(msrc[i] + min((int64_t)k0 * r + mchunk[i], m_last), dst);
      else
        dma16(msrc[i] + k0 + mchunk[i] * 8, dst);
    }
  };

#pragma unroll
  for (int st = 0; st < NST - 1; ++st) issue(st, min(st, KT - 1));
  wait_vm_barrier<(NST - 2) * PER_WAVE>();

  // one chain per parity of the 32-k block (the stage's slice sl) per chunk;
  // at a chunk's end tot += even + odd (the summation order of every shrink)
  f32x4 acc[2][2][NB], tot[2][NB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[h][g][b] = tot[g][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15;
  const int q = (lane >> 2) & 3, j = lane & 3;

  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt % NST;
    issue((kt + NST - 1) % NST, min(kt + NST - 1, KT - 1));
    const uint4* xt = lds + st * STAGE;
    const uint4* mt = xt + ST_XSLOTS;
#pragma unroll
    for (int sl = 0; sl < ST_KC / 32; ++sl) {
      const int ch = 4 * sl + (lane >> 4);   // logical chunk of this lane's fragments
      bf16x8 xa[2], mb[NB];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int row = wave * 32 + g * 16 + fr;
        xa[g] = as_bf16x8(xt[row * 8 + (ch ^ st_sw(row))]);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if constexpr (KM) {
          // rows k = 8 ch + {0..3} and {4..7} of the flat [64][r] slice; in
          // each 16-lane group, lane 4q + j addresses row 8 ch + q, ranks
          // 16 b + 4 j .. + 3, and receives rank 16 b + (lane & 15)
          const uint32_t off = (uint32_t)(((8 * ch + q) * r + 16 * b + 4 * j) * 2);
          const uint2 lo = tr_read(mt, off);
          const uint2 hi = tr_read(mt, off + (uint32_t)(4 * r * 2));
          mb[b] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        } else {
          const int c = b * 16 + fr;
          mb[b] = as_bf16x8(mt[c * 8 + (ch ^ st_sw(c))]);
        }
      }
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[sl][g][b] = mfma16(xa[g], mb[b], acc[sl][g][b]);
    }
    wait_vm_barrier<(NST - 2) * PER_WAVE>();
    if ((kt + 1) % CST == 0 || kt + 1 == KT) {   // chunk end
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
          for (int i = 0; i < 4; ++i) tot[g][b][i] = tot[g][b][i] + (acc[0][g][b][i] + acc[1][g][b][i]);
          acc[0][g][b] = acc[1][g][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

  // tot[g][b][i] = T[32 wave + 16 g + 4 (lane / 16) + i][16 b + lane % 16]
  float* red = (float*)lds;  // [ST_TM][64]
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(wave * 32 + g * 16 + 4 * (lane >> 4) + i) * 64 + b * 16 + (lane & 15)] = tot[g][b][i];
  __syncthreads();
  auto val = [&](int row, int c) { return red[row * 64 + c]; };
  shrink_emit(val, out, 0, r, scale, rm, p0, rows, ST_TM, plane, r_max);
  if (!KM && sec.mat) shrink_emit(val, sec.out, sec.c2, sec.r, sec.scale, rm, p0, rows, ST_TM, plane, r_max);
}

// One block per CU.  Blocks take the work items XCD-contiguously -- the
// adapter tiles (32 rows, or 128 with TALL; pre[n_ad] of them), each cut into
// n_parts ranges of the nch k chunks (n_parts > 1: 32-row tiles only, chunk
// sums to part[tile][chunk][32][64], folded by shrink_fold_kernel) -- then
// zero, grid-stride, the rows of tokens that belong to no active adapter
// (adpos == -1), and block 0 clears `zero`.
template <bool TALL>
__global__ __launch_bounds__(256) void shrink_kernel(
    const uint16_t* __restrict__ in, int64_t ld_in, int K, const uint16_t* __restrict__ mat_pack,
    int from_b, const lora_adapter_desc* __restrict__ desc, const int32_t* __restrict__ adpos,
    const ShrinkRows rm, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ pre32, int n_ad, int64_t n_tokens, uint16_t* __restrict__ out,
    int r_max, uint4* __restrict__ zero, const uint16_t* __restrict__ mat_pack2,
    const lora_adapter_desc* __restrict__ desc2, uint16_t* __restrict__ out2, int n_parts,
    int nch, float* __restrict__ part) {
  extern __shared__ uint4 sh_lds[];
  const int tid = threadIdx.x;
  const int64_t plane = n_tokens * r_max;
  const ItemRange ir = xcd_items(pre32[n_ad] * n_parts);
  for (int item = ir.first; item < ir.end; item += ir.step) {
    const int tile = item / n_parts, pp = item - tile * n_parts;
    const int c0 = pp * nch / n_parts, c1 = (pp + 1) * nch / n_parts;
    float* pt = n_parts > 1 ? part + (size_t)tile * nch * (SH_TM * 64) : nullptr;
    TileInfo ti;
    tile_of(pre32, offsets, n_ad, tile, TALL ? ST_TM : SH_TM, ti);
    const lora_adapter_desc d = desc[ti.a];
    const int r = d.rank;
    const uint16_t* mat = mat_pack + (from_b ? d.b_off : d.a_off);
    int nb = (r + 15) / 16;
    const float sc = d.scale;
    ShrinkSecond sec{nullptr, 0, 0, 0.f, out2};
    if (mat_pack2) {   // dual (A factors only; the host keeps both ranks <= 32)
      const lora_adapter_desc d2 = desc2[ti.a];
      sec.mat = mat_pack2 + d2.a_off;
      sec.r = d2.rank;
      sec.c2 = 16 * nb;
      sec.scale = d2.scale;
      nb += (d2.rank + 15) / 16;
    }
    __syncthreads();   // the previous item's LDS reads are done before the ring refills
#define SHRINK_TILE(NB, KM)                                                                    \
  do {                                                                                         \
    if constexpr (TALL)                                                                        \
      shrink_tall_tile<NB, KM>(in, ld_in, K, mat, r, sc, sec, rm, ti.p0, ti.rows, sh_lds, out, \
                               plane, r_max);                                                  \
    else                                                                                       \
      shrink_tile<NB, KM>(in, ld_in, K, mat, r, sc, sec, rm, ti.p0, ti.rows, sh_lds, out,      \
                          plane, r_max, c0, c1, pt);                                           \
  } while (0)
    if (from_b) {
      if (nb == 1) SHRINK_TILE(1, true);
      else if (nb == 2) SHRINK_TILE(2, true);
      else if (nb == 3) SHRINK_TILE(3, true);
      else SHRINK_TILE(4, true);
    } else {
      if (nb == 1) SHRINK_TILE(1, false);
      else if (nb == 2) SHRINK_TILE(2, false);
      else if (nb == 3) SHRINK_TILE(3, false);
      else SHRINK_TILE(4, false);
    }
#undef SHRINK_TILE
  }
  if (blockIdx.x == 0 && zero != nullptr && tid < 16) zero[tid] = make_uint4(0, 0, 0, 0);
  for (int64_t p = (int64_t)blockIdx.x * 256 + tid; p < n_tokens; p += (int64_t)gridDim.x * 256) {
    if (adpos[p] >= 0) continue;
    const int64_t orow = rm.out ? rm.out[p] : p;
    for (int k = 0; k < (out2 ? 2 : 1); ++k) {
      uint16_t* ob = k ? out2 : out;
      uint4* o = (uint4*)(ob + orow * r_max);
      uint4* ol = (uint4*)(ob + plane + orow * r_max);
      for (int c = 0; c < r_max / 8; ++c) o[c] = ol[c] = make_uint4(0, 0, 0, 0);
    }
  }
}

// After a split shrink: per 32-row tile, T = fold of its nch chunk sums in
// chunk order, scaled and split into the planes exactly as an unsplit tile
// does it (shrink_emit), for the first table and, dual, the second.
__global__ __launch_bounds__(256) void shrink_fold_kernel(
    const float* __restrict__ part, int nch, const lora_adapter_desc* __restrict__ desc,
    const ShrinkRows rm, const int32_t* __restrict__ offsets, const int32_t* __restrict__ pre32,
    int n_ad, int64_t n_tokens, uint16_t* __restrict__ out, int r_max,
    const lora_adapter_desc* __restrict__ desc2, uint16_t* __restrict__ out2) {
  const int64_t plane = n_tokens * r_max;
  const ItemRange ir = xcd_items(pre32[n_ad]);
  for (int tile = ir.first; tile < ir.end; tile += ir.step) {
    TileInfo ti;
    tile_of(pre32, offsets, n_ad, tile, SH_TM, ti);
    const lora_adapter_desc d = desc[ti.a];
    const float* pt = part + (size_t)tile * nch * (SH_TM * 64);
    auto val = [&](int row, int c) {
      float t = 0.f;
      for (int ch = 0; ch < nch; ++ch) t = t + pt[(size_t)ch * (SH_TM * 64) + row * 64 + c];
      return t;
    };
    shrink_emit(val, out, 0, d.rank, d.scale, rm, ti.p0, ti.rows, SH_TM, plane, r_max);
    if (desc2) {
      const lora_adapter_desc d2 = desc2[ti.a];
      shrink_emit(val, out2, 16 * ((d.rank + 15) / 16), d2.rank, d2.scale, rm, ti.p0, ti.rows,
                  SH_TM, plane, r_max);
    }
  }
}

// ------------------------------------------------------------------ grad
constexpr int GR_TC = 1024;   // tokens per chunk (per-adapter split for balance)
constexpr int GR_TT = 32;     // tokens per stage
constexpr int GR_NJ = 256;    // output columns per block
constexpr int GR_QSLOTS = GR_TT * 32;   // 32 token rows x 512 B of Q
constexpr int GR_QDMA = 4;              // Q DMA instructions per wave per stage
// The P tile of a stage holds both bf16 planes (hi, lo) of 32 tokens, each
// token row 4*PN 16-byte chunks wide (PN = 1: ranks <= 32, PN = 2: <= 64).
template <int PN> struct GrP {
  static constexpr int PW = 4 * PN;                 // chunks per token row
  static constexpr int SLOTS = 2 * GR_TT * PW;      // 256 * PN
  static constexpr int STAGE = GR_QSLOTS + SLOTS;
  static constexpr int PER_WAVE = GR_QDMA + PN;     // DMA instructions per wave per stage
  static constexpr int NST = 5;                     // ring depth (deeper measured no faster)
  // pair (32-byte) swizzle: the 8 token rows that one transposing read of 32
  // lanes touches (t0..t0+3 and t0+8..t0+11) land on distinct banks
  static __device__ __forceinline__ int sw(int t) {
    return PN == 1 ? ((t >> 3) & 1) : (((t >> 1) & 1) | (((t >> 3) & 1) << 1));
  }
};

// Q tile swizzle: chunk c of token row t is stored at c ^ fq(t).  A transposed
// 8-byte read (ds_read_b64_tr_b16) by 16 lanes touches 4 consecutive rows x
// 32 B; fq spreads those rows (and the rows of the next 16-lane group, 8 rows
// further) over distinct banks.
__device__ __forceinline__ int gr_fq(int t) { return (2 * (t & 3)) | (8 * ((t >> 3) & 1)); }

// T[c][j] = sum_{t in chunk} P[t][c] Q[t][j] for one chunk of one adapter and
// 256 columns j.  P is the scaled per-token vector stored as two bf16 planes
// (hi, lo; hi + lo carries ~16 bits), so both MFMA operands are bf16 and the
// product is exact up to fp32 accumulation.  MFMA K is the token axis: each
// 32-token stage is one v_mfma_f32_16x16x32 per (16 columns, 16 ranks, plane).
// Both operands come from row-major LDS tiles through the transposing read: in
// a 16-lane group, lane 4q + b addresses row (t0 + q), columns 4b..4b+3, and
// lane i receives column i of rows t0..t0+3.  Tokens past the chunk end read a
// zero row for P, so they add nothing.
// mode 0 (dB): out layout [D][r] (c fastest): MFMA M = c, N = j.
// mode 1 (dA): out layout [r][D] (j fastest): MFMA M = j, N = c.
// Dual P (mode 1): a second set of planes at element offset p2_off from P,
// with the same row stride r_max; tile ranks [r_max, 2 r_max) come from it.
// nblk column blocks (j0, j0 + 256, ..) stream as one sequence of stages
// (the token stages of each block in turn), so the ring does not drain between
// blocks; after a block's last stage write(j0 of the block) stores acc, which
// then restarts from zero.
// (MULTI = false: one block, the plain loop.)
template <int NCB, int MODE, int PN, bool MULTI, class F>
__device__ __forceinline__ void grad_tile(const uint16_t* __restrict__ P, int64_t plane, int r_max,
                                          int64_t p2_off, const uint16_t* __restrict__ zero,
                                          const uint16_t* __restrict__ Q, int64_t ld_q, int D,
                                          const int32_t* tok_s, int p_base, int rows, int j0,
                                          int nblk_, uint4* lds, f32x4 (&acc)[4][4], F&& write) {
  using G = GrP<PN>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int KT = (rows + GR_TT - 1) / GR_TT;
  const int nblk = MULTI ? nblk_ : 1;
  const int total = nblk * KT;
  // DMA sources.  Q: instruction i of wave w fills rows (4w + i)*2 + L/32,
  // chunk L%32.  P: slot s = (w*PN + i)*64 + L holds plane s / (32*PW), token
  // row (s / PW) % 32, physical chunk s % PW.
  int qrow[GR_QDMA], qcol[GR_QDMA];   // qcol: column within the 256-column block
#pragma unroll
  for (int i = 0; i < GR_QDMA; ++i) {
    const int row = (wave * GR_QDMA + i) * 2 + (lane >> 5);
    qrow[i] = row;
    qcol[i] = ((lane & 31) ^ gr_fq(row)) * 8;
  }
  int prow[PN];
  int64_t poff[PN];
  int pzoff[PN];
  const int pchunks = (p2_off ? 2 : 1) * (r_max / 8);   // 16-byte chunks per token row
#pragma unroll
  for (int i = 0; i < PN; ++i) {
    const int s = (wave * PN + i) * 64 + lane;
    const int pl = s / (GR_TT * G::PW);
    const int t = (s / G::PW) % GR_TT;
    const int c = min((s % G::PW) ^ (2 * G::sw(t)), pchunks - 1);
    const bool second = c >= r_max / 8;
    prow[i] = t;
    poff[i] = pl * plane + (second ? p2_off + (c - r_max / 8) * 8 : c * 8);
    pzoff[i] = c * 8;
  }
  auto issue = [&](int st, int sq) {   // stage sq of the sequence into ring slot st
    uint4* base = lds + st * G::STAGE;
    const int blk = MULTI ? sq / KT : 0;
    const int t0 = (sq - blk * KT) * GR_TT;
    const int jb = j0 + blk * GR_NJ;
    int qt[GR_QDMA], pt[PN];
#pragma unroll
    for (int i = 0; i < GR_QDMA; ++i) qt[i] = tok_s[min(t0 + qrow[i], rows - 1)];
#pragma unroll
    for (int i = 0; i < PN; ++i) {
      // P row: the chunk's token (tok_s) or, with p_base >= 0, the position itself
      const int tp = p_base >= 0 ? p_base + min(t0 + prow[i], rows - 1)
                                 : tok_s[min(t0 + prow[i], rows - 1)];   // unconditional: no branch
      pt[i] = t0 + prow[i] < rows ? tp : -1;
    }
#pragma unroll
    for (int i = 0; i < GR_QDMA; ++i)
      dma16(Q + (int64_t)qt[i] * ld_q + min(jb + qcol[i], D - 8),
            __builtin_amdgcn_readfirstlane(lds_u32(base + (wave * GR_QDMA + i) * 64)));
#pragma unroll
    for (int i = 0; i < PN; ++i) {
      const uint16_t* g = pt[i] >= 0 ? P + (int64_t)pt[i] * r_max + poff[i] : zero + pzoff[i];
      dma16(g, __builtin_amdgcn_readfirstlane(lds_u32(base + GR_QSLOTS + (wave * PN + i) * 64)));
    }
  };

#pragma unroll
  for (int st = 0; st < G::NST - 1; ++st) issue(st, min(st, total - 1));
  wait_vm_barrier<(G::NST - 2) * G::PER_WAVE>();

  const int g16 = lane >> 4;   // 16-lane group: tokens 8*g16 .. 8*g16+7 of the stage
  const int li = lane & 15;
  int sq = 0;
  for (int blk = 0; blk < nblk; ++blk) {
  for (int kt = 0; kt < KT; ++kt, ++sq) {
    const int st = sq % G::NST;
    issue((sq + G::NST - 1) % G::NST, min(sq + G::NST - 1, total - 1));
    const uint4* qt = lds + st * G::STAGE;
    const uint4* ptile = qt + GR_QSLOTS;
    // Q fragments: 4 column sub-tiles of this wave's 64 columns
    bf16x8 qf[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      uint2 hv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 8 * g16 + 4 * h + (li >> 2);
        const int jl = wave * 64 + jt * 16 + 4 * (li & 3);
        const uint32_t off = t * 512 + (((jl >> 3) ^ gr_fq(t)) << 4) + ((jl & 7) << 1);
        hv[h] = tr_read(qt, off);
      }
      qf[jt] = as_bf16x8(make_uint4(hv[0].x, hv[0].y, hv[1].x, hv[1].y));
    }
    // P fragments (both planes): tokens 8*g16 .. +7, rank column cb*16 + li
    bf16x8 pf[2][NCB];
#pragma unroll
    for (int pl = 0; pl < 2; ++pl)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        uint2 hv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int t = 8 * g16 + 4 * h + (li >> 2);
          const int col = cb * 16 + 4 * (li & 3);
          const int pc = (col >> 3) ^ (2 * G::sw(t));
          const uint32_t off = ((pl * GR_TT + t) * G::PW + pc) * 16 + ((col & 7) << 1);
          hv[h] = tr_read(ptile, off);
        }
        pf[pl][cb] = as_bf16x8(make_uint4(hv[0].x, hv[0].y, hv[1].x, hv[1].y));
      }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        if (MODE == 0) {
          acc[jt][cb] = mfma16(pf[0][cb], qf[jt], acc[jt][cb]);
          acc[jt][cb] = mfma16(pf[1][cb], qf[jt], acc[jt][cb]);
        } else {
          acc[jt][cb] = mfma16(qf[jt], pf[0][cb], acc[jt][cb]);
          acc[jt][cb] = mfma16(qf[jt], pf[1][cb], acc[jt][cb]);
        }
      }
    wait_vm_barrier<(G::NST - 2) * G::PER_WAVE>();
  }
  // the block's last token stage is done (the next block's first stages are
  // in flight): store it and start the next one from zero
  write(j0 + blk * GR_NJ);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA may outlive the block
}

// Second table of a dual (mode 1) reduction: ranks [r_max, 2 r_max) of the
// tile are T for desc2 / out2 (P planes at p2_off); off when desc2 is null.
struct GradDual {
  const lora_adapter_desc* desc2;
  float* out2;
  int64_t p2_off;
};

template <int MODE, int PN, bool MULTI>
__device__ __forceinline__ void grad_item(
    const uint16_t* __restrict__ P, int64_t plane, int r_max, const uint16_t* __restrict__ zero,
    const uint16_t* __restrict__ Q, int64_t ld_q, int D,
    const lora_adapter_desc* __restrict__ desc, const int32_t* __restrict__ q_rows, int p_ident,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ chunk_pre, int n_ad,
    float* __restrict__ out_pack, float* __restrict__ partial, int accumulate, int slot, int j0,
    int nblk, int32_t* tok_s, uint4* gr_lds, const GradDual du) {
  TileInfo ti;
  tile_of<false>(chunk_pre, offsets, n_ad, slot, GR_TC, ti);
  __syncthreads();   // every wave is done with the previous item's tokens and ring
  for (int i = threadIdx.x; i < ti.rows; i += 256) tok_s[i] = q_rows ? q_rows[ti.p0 + i] : ti.p0 + i;
  const int p_base = p_ident ? ti.p0 : -1;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const lora_adapter_desc d = desc[ti.a];
  const int r = d.rank;
  const bool dual = MODE == 1 && du.desc2 != nullptr;
  const lora_adapter_desc d2 = dual ? du.desc2[ti.a] : d;
  const int nchunks = chunk_pre[ti.a + 1] - chunk_pre[ti.a];
  const int rt = dual ? 2 * r_max : r_max;   // tile ranks (partial row count)
  const int64_t p2 = dual ? du.p2_off : 0;

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ncb = dual ? (r_max + d2.rank + 15) / 16 : (r + 15) / 16;

  // ---- write of one 256-column block.  Region of this adapter: D*r floats.
  const int64_t base = MODE == 0 ? d.b_off : d.a_off;
  const bool direct = nchunks == 1;
  float* dst = direct ? out_pack + base : partial + (int64_t)slot * D * rt;
  // dual, direct: ranks >= r_max go to the second table's region
  float* dst2 = direct && dual ? du.out2 + d2.a_off : nullptr;
  auto write = [&](int jb) {
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (ct >= ncb) continue;
        if (MODE == 0) {
          // D[c][j]: lane holds c = ct*16 + 4*(lane/16) + i, j = jt*16 + lane%16
          const int c = ct * 16 + 4 * (lane >> 4);
          const int j = jb + wave * 64 + jt * 16 + (lane & 15);
          if (c >= r || j >= D) continue;
          float4* p = (float4*)(dst + (int64_t)j * r + c);
          float4 v = make_float4(acc[jt][ct][0], acc[jt][ct][1], acc[jt][ct][2], acc[jt][ct][3]);
          if (direct && accumulate) {
            float4 o = *p;
            v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
          }
          *p = v;
        } else {
          // D[j][c]: lane holds j = jt*16 + 4*(lane/16) + i, c = ct*16 + lane%16
          const int j = jb + wave * 64 + jt * 16 + 4 * (lane >> 4);
          const int c = ct * 16 + (lane & 15);
          const bool hi = dual && c >= r_max;   // rank c - r_max of the second table
          if ((hi ? c - r_max >= d2.rank : c >= r) || j >= D) continue;
          float4* p = (float4*)(hi && direct ? dst2 + (int64_t)(c - r_max) * D + j
                                             : dst + (int64_t)c * D + j);
          float4 v = make_float4(acc[jt][ct][0], acc[jt][ct][1], acc[jt][ct][2], acc[jt][ct][3]);
          if (direct && accumulate) {
            float4 o = *p;
            v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
          }
          *p = v;
        }
      }
  };
#define GRAD_TILE(NCB)                                                                       \
  grad_tile<NCB, MODE, PN, MULTI>(P, plane, r_max, p2, zero, Q, ld_q, D, tok_s, p_base,         \
                                  ti.rows, j0, nblk, gr_lds, acc, write)
  if (PN == 1) {
    if (ncb == 1) GRAD_TILE(1);
    else GRAD_TILE(2);
  } else {
    if (ncb == 1) GRAD_TILE(1);
    else if (ncb == 2) GRAD_TILE(2);
    else if (ncb == 3) GRAD_TILE(3);
    else GRAD_TILE(4);
  }
#undef GRAD_TILE
}

// One block per CU.  Items are (gradient chunk, group of cpi 256-column
// blocks) pairs, column groups fastest (the groups of a chunk read the same
// token rows), taken XCD-contiguously.  Many small chunks (MoE segments of
// ~128 tokens) take whole rows of column blocks per item (cpi = all), so an
// item's fixed costs (its token ids, the ring's first stages) are paid once
// per chunk rather than once per 256 columns.
template <int MODE, int PN, bool MULTI>
__global__ __launch_bounds__(256) void grad_kernel(
    const uint16_t* __restrict__ P, int64_t plane, int r_max, const uint16_t* __restrict__ zero,
    const uint16_t* __restrict__ Q, int64_t ld_q, int D,
    const lora_adapter_desc* __restrict__ desc, const int32_t* __restrict__ q_rows, int p_ident,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ chunk_pre, int n_ad,
    float* __restrict__ out_pack, float* __restrict__ partial, int accumulate, GradDual du,
    int cpi) {
  extern __shared__ uint4 gr_lds[];
  // the chunk's token ids, cached in LDS: the DMA loop may issue no
  // compiler-tracked global loads (their waits would also wait for the DMA)
  __shared__ int32_t tok_s[GR_TC];
  const int ncol = (D + GR_NJ - 1) / GR_NJ;
  const int ngrp = (ncol + cpi - 1) / cpi;
  const ItemRange ir = xcd_items(chunk_pre[n_ad] * ngrp);
  for (int item = ir.first; item < ir.end; item += ir.step) {
    const int slot = item / ngrp;
    const int g = item - slot * ngrp;
    grad_item<MODE, PN, MULTI>(P, plane, r_max, zero, Q, ld_q, D, desc, q_rows, p_ident,
                               offsets, chunk_pre, n_ad, out_pack, partial, accumulate, slot,
                               g * cpi * GR_NJ, min(cpi, ncol - g * cpi), tok_s, gr_lds, du);
  }
}

// One reduction of a paired launch (both over the same segments).
struct GradSide {
  const uint16_t* P;
  const uint16_t* Q;
  int64_t ld_q;
  int D;
  const lora_adapter_desc* desc;
  float* out_pack;
  float* partial;
};

// dB (mode 0) and dA (mode 1) of one layer in one launch: items of the first
// side, then of the second, spread XCD-contiguously as in grad_kernel.  Both
// sides share the segments, the plane stride and the rank bound.
template <int PN, bool MULTI>
__global__ __launch_bounds__(256) void grad_pair_kernel(
    GradSide s0, GradSide s1, int64_t plane, int r_max, const uint16_t* __restrict__ zero,
    const int32_t* __restrict__ q_rows, int p_ident, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ chunk_pre, int n_ad, int accumulate, int cpi) {
  extern __shared__ uint4 gr_lds[];
  __shared__ int32_t tok_s[GR_TC];
  const int nc0 = (s0.D + GR_NJ - 1) / GR_NJ, nc1 = (s1.D + GR_NJ - 1) / GR_NJ;
  const int ng0 = (nc0 + cpi - 1) / cpi, ng1 = (nc1 + cpi - 1) / cpi;
  const int n0 = chunk_pre[n_ad] * ng0;
  const ItemRange ir = xcd_items(n0 + chunk_pre[n_ad] * ng1);
  const GradDual none{nullptr, nullptr, 0};
  for (int item = ir.first; item < ir.end; item += ir.step) {
    if (item < n0) {
      const int slot = item / ng0, g = item - slot * ng0;
      grad_item<0, PN, MULTI>(s0.P, plane, r_max, zero, s0.Q, s0.ld_q, s0.D, s0.desc, q_rows,
                              p_ident, offsets, chunk_pre, n_ad, s0.out_pack, s0.partial,
                              accumulate, slot, g * cpi * GR_NJ, min(cpi, nc0 - g * cpi), tok_s,
                              gr_lds, none);
    } else {
      const int it = item - n0, slot = it / ng1, g = it - slot * ng1;
      grad_item<1, PN, MULTI>(s1.P, plane, r_max, zero, s1.Q, s1.ld_q, s1.D, s1.desc, q_rows,
                              p_ident, offsets, chunk_pre, n_ad, s1.out_pack, s1.partial,
                              accumulate, slot, g * cpi * GR_NJ, min(cpi, nc1 - g * cpi), tok_s,
                              gr_lds, none);
    }
  }
}

// Slice blockIdx.y of one key's result (grid y: blocks over D*r_max/1024).
// Sums the chunk partials of adapters with several chunks, in chunk order;
// with accumulate == 0 writes zeros for active adapters that own no token.
__device__ __forceinline__ void grad_finalize_body(
    int a, const lora_adapter_desc* __restrict__ desc, const uint8_t* __restrict__ active,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ chunk_pre, int D,
    int64_t slot_floats, int mode, float* __restrict__ out_pack, const float* __restrict__ partial,
    int accumulate) {
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
        const float4 p = *(const float4*)(partial + (int64_t)(s0 + q) * slot_floats + e);
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

// Block (x, y) finalizes slice y of keys [x kpb, (x + 1) kpb) (kpb <= 256):
// the block's threads first check one key each, so that a group of keys with
// nothing to do (one chunk, or tokens and no zero fill) costs one round of
// loads; the keys with work are then done in key order.
__device__ __forceinline__ void grad_finalize_keys(
    int a0, int kpb, int n_ad, const lora_adapter_desc* __restrict__ desc,
    const uint8_t* __restrict__ active, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ chunk_pre, int D, int64_t slot_floats, int mode,
    float* __restrict__ out_pack, const float* __restrict__ partial, int accumulate) {
  if (kpb == 1) {   // one key per block: its own early exits are the check
    grad_finalize_body(a0, desc, active, offsets, chunk_pre, D, slot_floats, mode, out_pack,
                       partial, accumulate);
    return;
  }
  __shared__ uint64_t s_work[4];   // bit k: key a0 + k has work
  const int k = threadIdx.x, a = a0 + k;
  bool work = false;
  if (k < kpb && a < n_ad && active[a]) {
    const bool empty = offsets[a + 1] == offsets[a];
    work = (empty && !accumulate) || (!empty && chunk_pre[a + 1] - chunk_pre[a] >= 2);
  }
  const uint64_t bal = __ballot(work);
  if ((k & 63) == 0) s_work[k >> 6] = bal;
  __syncthreads();
  for (int w = 0; w < 4; ++w)
    for (uint64_t m = s_work[w]; m; m &= m - 1)
      grad_finalize_body(a0 + 64 * w + __ffsll((long long)m) - 1, desc, active, offsets,
                         chunk_pre, D, slot_floats, mode, out_pack, partial, accumulate);
}

__global__ __launch_bounds__(256) void grad_finalize_kernel(
    const lora_adapter_desc* __restrict__ desc, const uint8_t* __restrict__ active,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ chunk_pre, int n_ad,
    int kpb, int D, int64_t slot_floats, int mode, float* __restrict__ out_pack,
    const float* __restrict__ partial, int accumulate) {
  grad_finalize_keys(blockIdx.x * kpb, kpb, n_ad, desc, active, offsets, chunk_pre, D,
                     slot_floats, mode, out_pack, partial, accumulate);
}

// Both sides of a paired launch: blocks x < nb0 finalize side 0 (mode 0), the
// rest side 1 (mode 1).
__global__ __launch_bounds__(256) void grad_finalize_pair_kernel(
    GradSide s0, GradSide s1, const uint8_t* __restrict__ active,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ chunk_pre, int n_ad,
    int kpb, int nb0, int r_max, int accumulate) {
  const int x = blockIdx.x;
  if (x < nb0)
    grad_finalize_keys(x * kpb, kpb, n_ad, s0.desc, active, offsets, chunk_pre, s0.D,
                       (int64_t)s0.D * r_max, 0, s0.out_pack, s0.partial, accumulate);
  else
    grad_finalize_keys((x - nb0) * kpb, kpb, n_ad, s1.desc, active, offsets, chunk_pre, s1.D,
                       (int64_t)s1.D * r_max, 1, s1.out_pack, s1.partial, accumulate);
}

}  // namespace lora

namespace lora_host {
using namespace lora;

// Blocks of a one-block-per-CU grid: the device's CU count rounded down to a
// multiple of 8 (one stretch per XCD).
static unsigned persistent_blocks() { return (unsigned)(std::max(device_cus(), 8) & ~7); }

// Parts per 32-row tile of a K-split shrink: about 256 / (bound on the tiles)
// when that bound is at most 128 (n_tokens / 32 + n_ad, one partial tile per
// adapter), capped by the number of k chunks; else 1.  A fixed 256, not the
// device's CU count, so that workspace sizes do not depend on the device.
int shrink_split_parts(int64_t n_tokens, int n_ad, int K) {
  const int nch = (K + SHRINK_KCH - 1) / SHRINK_KCH;
  const int64_t tiles = (n_tokens + SH_TM - 1) / SH_TM + n_ad;
  if (n_tokens <= 0 || nch < 2 || tiles > 128) return 1;
  return (int)std::min<int64_t>(nch, (256 + tiles - 1) / tiles);
}

size_t shrink_part_floats(int64_t n_tokens, int n_ad, int K) {
  if (shrink_split_parts(n_tokens, n_ad, K) <= 1) return 0;
  const int64_t tiles = (n_tokens + SH_TM - 1) / SH_TM + n_ad;
  return (size_t)tiles * ((K + SHRINK_KCH - 1) / SHRINK_KCH) * SH_TM * 64;
}

lora_status launch_shrink(const uint16_t* in, int64_t ld_in, int K, const uint16_t* mat_pack,
                          int from_b, const lora_adapter_desc* desc, const int32_t* adpos,
                          const int32_t* in_rows, const int32_t* out_rows, const float* rowscale,
                          const int32_t* offsets, const int32_t* pre32, int n_ad,
                          int64_t n_tokens, uint16_t* out, int r_max, void* zero, hipStream_t s,
                          const uint16_t* mat_pack2, const lora_adapter_desc* desc2,
                          uint16_t* out2, const int32_t* pre128, float* part,
                          size_t part_floats) {
  if (n_tokens <= 0) return LORA_OK;
  if (mat_pack2 && (from_b || r_max > 32 || !desc2 || !out2)) {
    set_error("shrink: a dual shrink takes two A tables with ranks <= 32");
    return LORA_E_INVALID_ARG;
  }
  const int nb_max = (mat_pack2 ? 2 : 1) * ((r_max + 15) / 16);
  // 128-row tiles once the batch gives every CU at least half of one (16384
  // rows on 256 CUs: measured 6% faster there and 8% at 32768; at 8192 rows,
  // a quarter tile per CU, the 32-row tiles keep every CU busy and win by 40%)
  const bool tall = pre128 != nullptr && 2 * n_tokens >= (int64_t)ST_TM * persistent_blocks() &&
                    K % ST_KC == 0;
  size_t lds;
  if (tall) {
    lds = (size_t)ST_TM * 64 * sizeof(float);
    for (int nb = 1; nb <= nb_max; ++nb)
      lds = std::max(lds, (size_t)ST_NST * (ST_XSLOTS + (nb <= 2 ? 2 : 4) * 128) * 16);
  } else {
    // the ring, then the odd chains' hand-over area [SH_TM][64] floats
    const size_t ring[4] = {(size_t)sh_nst<1>() * (SH_XSLOTS + 256) * 16,
                            (size_t)sh_nst<2>() * (SH_XSLOTS + 512) * 16,
                            (size_t)sh_nst<3>() * (SH_XSLOTS + 768) * 16,
                            (size_t)sh_nst<4>() * (SH_XSLOTS + 1024) * 16};
    lds = ring[nb_max - 1] + (size_t)SH_TM * 64 * sizeof(float);
  }
  // K split (32-row tiles, when the tiles alone leave most CUs idle): parts of
  // the k chunks per tile, so that tiles x parts covers about every CU
  const int nch = (K + SHRINK_KCH - 1) / SHRINK_KCH;
  int n_parts = 1;
  if (!tall && part) {
    n_parts = shrink_split_parts(n_tokens, n_ad, K);
    if (n_parts > 1 &&
        part_floats < shrink_part_floats(n_tokens, n_ad, K))
      n_parts = 1;
  }
  auto go = [&](auto tall_) -> lora_status {
    constexpr bool T = decltype(tall_)::value;
    // the dynamic LDS bound, raised once to the largest ring this kernel takes
    // (a thread-safe one-time initialisation, then read-only)
    static const hipError_t attr_err = hipFuncSetAttribute(
        (const void*)shrink_kernel<T>, hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)(T ? std::max((size_t)ST_TM * 64 * sizeof(float),
                           (size_t)ST_NST * (ST_XSLOTS + 4 * 128) * 16)
                : (size_t)sh_nst<4>() * (SH_XSLOTS + 1024) * 16 + (size_t)SH_TM * 64 * 4));
    TRY_HIP(attr_err);
    const ShrinkRows rmap{in_rows, out_rows, rowscale};
    hipLaunchKernelGGL(shrink_kernel<T>, dim3(persistent_blocks()), dim3(256), lds, s, in, ld_in,
                       K, mat_pack, from_b, desc, adpos, rmap, offsets, T ? pre128 : pre32, n_ad,
                       n_tokens, out, r_max, (uint4*)zero, mat_pack2, desc2, out2, n_parts, nch,
                       part);
    const lora_status st = launch_check("shrink");
    if (st != LORA_OK || n_parts == 1) return st;
    hipLaunchKernelGGL(shrink_fold_kernel, dim3(persistent_blocks()), dim3(256), 0, s, part, nch,
                       desc, rmap, offsets, pre32, n_ad, n_tokens, out, r_max,
                       mat_pack2 ? desc2 : nullptr, out2);
    return launch_check("shrink_fold");
  };
  return tall ? go(std::true_type{}) : go(std::false_type{});
}

// Keys per finalize block: 256 when the keys average under a quarter of a
// gradient chunk of tokens (most have one chunk and nothing to fold, so a
// block checks many; at most a quarter of them can have several chunks), else
// 1 (every key's chunk partials get blocks of their own).
static int finalize_keys_per_block(int64_t n_tokens, int n_ad) {
  return n_tokens < (int64_t)n_ad * (GR_TC / 4) ? 256 : 1;
}

// 256-column blocks per gradient item: all of them (one item per chunk) when
// the chunks alone give every CU a few items, else one.  Chunks are about one
// per key and one per 1024 tokens.
static int grad_cols_per_item(int64_t n_tokens, int n_ad, int D) {
  const int64_t chunks = std::min<int64_t>(n_ad, n_tokens) + n_tokens / GR_TC;
  const int ncol = (D + GR_NJ - 1) / GR_NJ;
  return chunks >= 2 * (int64_t)persistent_blocks() ? ncol : 1;
}

template <int MODE, int PN, bool MULTI>
lora_status launch_grad_t(dim3 grid, const uint16_t* P, int64_t plane, int r_max,
                          const uint16_t* zero, const uint16_t* Q, int64_t ld_q, int D,
                          const lora_adapter_desc* desc, const int32_t* q_rows, int p_ident,
                          const int32_t* offsets, const int32_t* chunk_pre, int n_ad,
                          float* out_pack, float* partial, int accumulate, GradDual du, int cpi,
                          hipStream_t s) {
  const size_t lds = (size_t)GrP<PN>::NST * GrP<PN>::STAGE * sizeof(uint4);
  static const hipError_t attr_err = hipFuncSetAttribute(
      (const void*)grad_kernel<MODE, PN, MULTI>, hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)lds);   // once, thread-safely
  TRY_HIP(attr_err);
  hipLaunchKernelGGL((grad_kernel<MODE, PN, MULTI>), grid, dim3(256), lds, s, P, plane, r_max,
                     zero, Q,
                     ld_q, D, desc, q_rows, p_ident, offsets, chunk_pre, n_ad, out_pack, partial,
                     accumulate, du, cpi);
  return launch_check("grad");
}

lora_status launch_grad(int mode, const uint16_t* P, int r_max, const void* zero,
                        const uint16_t* Q, int64_t ld_q, int D, const lora_adapter_desc* desc,
                        const uint8_t* active, const int32_t* q_rows, int p_ident,
                        const int32_t* offsets, const int32_t* chunk_pre, int n_ad,
                        int64_t n_tokens, float* out_pack, float* partial, int accumulate,
                        hipStream_t s, const uint16_t* P2, const lora_adapter_desc* desc2,
                        float* out2) {
  const bool dual = P2 != nullptr;
  if (dual && (mode != 1 || r_max > 32 || !desc2 || !out2)) {
    set_error("grad: a dual reduction takes two mode-1 tables with ranks <= 32");
    return LORA_E_INVALID_ARG;
  }
  const int rt = dual ? 2 * r_max : r_max;   // tile ranks
  if (n_tokens > 0) {
    dim3 grid(persistent_blocks());
    const int64_t plane = n_tokens * r_max;
    const uint16_t* z = (const uint16_t*)zero;
    const GradDual du{desc2, out2, dual ? (int64_t)(P2 - P) : 0};
    lora_status st;
    const int cpi = grad_cols_per_item(n_tokens, n_ad, D);
#define LAUNCH_GRAD(M, PN)                                                                   \
  (cpi > 1 ? launch_grad_t<M, PN, true>(grid, P, plane, r_max, z, Q, ld_q, D, desc, q_rows,  \
                                         p_ident, offsets, chunk_pre, n_ad, out_pack, partial, \
                                         accumulate, du, cpi, s)                               \
           : launch_grad_t<M, PN, false>(grid, P, plane, r_max, z, Q, ld_q, D, desc, q_rows, \
                                          p_ident, offsets, chunk_pre, n_ad, out_pack,        \
                                          partial, accumulate, du, 1, s))
    if (rt <= 32)
      st = mode == 0 ? LAUNCH_GRAD(0, 1) : LAUNCH_GRAD(1, 1);
    else
      st = mode == 0 ? LAUNCH_GRAD(0, 2) : LAUNCH_GRAD(1, 2);
#undef LAUNCH_GRAD
    if (st) return st;
  }
  const int64_t slot = (int64_t)D * rt;   // floats per chunk partial
  const unsigned gy = (unsigned)std::max<int64_t>(1, std::min<int64_t>(64, cdiv((int64_t)D * r_max, 1024)));
  const int kpb = finalize_keys_per_block(n_tokens, n_ad);
  const unsigned gx = (unsigned)cdiv(n_ad, kpb);
  hipLaunchKernelGGL(grad_finalize_kernel, dim3(gx, gy), dim3(256), 0, s, desc, active, offsets,
                     chunk_pre, n_ad, kpb, D, slot, mode, out_pack, partial, accumulate);
  lora_status st = launch_check("grad_finalize");
  if (st || !dual) return st;
  hipLaunchKernelGGL(grad_finalize_kernel, dim3(gx, gy), dim3(256), 0, s, desc2, active, offsets,
                     chunk_pre, n_ad, kpb, D, slot, mode, out2, partial + (int64_t)r_max * D,
                     accumulate);
  return launch_check("grad_finalize");
}

lora_status launch_grad_pair(const uint16_t* u, const uint16_t* dy, int64_t ld_dy, int d_out,
                             float* dB_pack, float* partial_b, const uint16_t* v,
                             const uint16_t* x, int64_t ld_x, int d_in, float* dA_pack,
                             float* partial_a, int r_max, const void* zero,
                             const lora_adapter_desc* desc, const uint8_t* active,
                             const int32_t* q_rows, const int32_t* offsets,
                             const int32_t* chunk_pre, int n_ad, int64_t n_tokens, int accumulate,
                             hipStream_t s) {
  const GradSide s0{u, dy, ld_dy, d_out, desc, dB_pack, partial_b};
  const GradSide s1{v, x, ld_x, d_in, desc, dA_pack, partial_a};
  if (n_tokens > 0) {
    const int64_t plane = n_tokens * r_max;
    const uint16_t* z = (const uint16_t*)zero;
    const int cpi = grad_cols_per_item(n_tokens, n_ad, std::min(d_in, d_out));
    auto go = [&](auto pn, auto multi) -> lora_status {
      constexpr int PN = decltype(pn)::value;
      constexpr bool MULTI = decltype(multi)::value;
      const size_t lds = (size_t)GrP<PN>::NST * GrP<PN>::STAGE * sizeof(uint4);
      static const hipError_t attr_err = hipFuncSetAttribute(
          (const void*)grad_pair_kernel<PN, MULTI>, hipFuncAttributeMaxDynamicSharedMemorySize,
          (int)lds);   // once, thread-safely
      TRY_HIP(attr_err);
      hipLaunchKernelGGL((grad_pair_kernel<PN, MULTI>), dim3(persistent_blocks()), dim3(256), lds,
                         s, s0, s1, plane, r_max, z, q_rows, 0, offsets, chunk_pre, n_ad,
                         accumulate, MULTI ? cpi : 1);
      return launch_check("grad_pair");
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    const lora_status st =
        r_max <= 32 ? (cpi > 1 ? go(I1{}, std::true_type{}) : go(I1{}, std::false_type{}))
                    : (cpi > 1 ? go(I2{}, std::true_type{}) : go(I2{}, std::false_type{}));
    if (st) return st;
  }
  const unsigned gy = (unsigned)std::max<int64_t>(
      1, std::min<int64_t>(64, cdiv((int64_t)std::max(d_in, d_out) * r_max, 1024)));
  const int kpb = finalize_keys_per_block(n_tokens, n_ad);
  const int nb0 = (int)cdiv(n_ad, kpb);
  hipLaunchKernelGGL(grad_finalize_pair_kernel, dim3(2 * nb0, gy), dim3(256), 0, s, s0, s1,
                     active, offsets, chunk_pre, n_ad, kpb, nb0, r_max, accumulate);
  return launch_check("grad_finalize_pair");
}

int64_t grad_partial_floats(int64_t n_tokens, int n_ad, int64_t D, int r_max) {
  return (cdiv(n_tokens, GR_TC) + n_ad) * D * r_max;
}


}  // namespace lora_host
