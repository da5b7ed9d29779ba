// bf16 MFMA GEMM for gfx950: C[M][N] = sum_k A[m][k] * B[n][k] (both operands
// K-contiguous, fp32 accumulation), with three epilogues:
//   EPI_BF16  store bf16(C)                                  (base GEMMs, dh)
//   EPI_LSE   per-row (max, sum exp) over the tile's columns and the target
//             logit, for the lm_head online logsumexp        (token_logprobs)
//   EPI_GRAD  G = d (onehot(y) - exp(C - lse)) stored bf16   (logprob backward)
//
// Block tile 256 x 256, 512 threads = 8 waves (two per SIMD) in a 2 x 4 grid,
// each wave 128 x 64 as 4 x 2 tiles of v_mfma_f32_32x32x16_bf16 (128 fp32
// accumulators per lane).  Two waves per SIMD let one wave's epilogue, waits
// and LDS traffic overlap the other's MFMAs.  Operand tiles move global ->
// LDS by LDS-DMA into two stages of k = 64 (whole 128-byte lines per row:
// with 64-byte rows the texture path stalled on twice the requests, and the
// clock fell with it); all of the next stage's DMA issues in the first phase
// of a step (the first two stages in the prologue), one barrier per step.  LDS fragment reads run one 16-wide k
// slice ahead of the MFMAs.  LDS rows are 128 B with their 16-byte chunks
// XOR-swizzled (lds_sw) so the fragment reads of 16 consecutive rows hit
// distinct banks.  The MFMA computes the transposed sub-tile so that each
// lane ends with runs of 4 consecutive output columns (row reductions need
// one cross-lane step).  The bf16 epilogue stages the tile in the idle
// stages and writes whole 512-byte rows (scattered 16-byte stores of 32 rows
// per instruction cost ~10 us more per 8192x4096 output).  Tiles are ordered
// XCD-first (blocks are dispatched round-robin over the 8 XCDs, so each XCD
// gets a contiguous tile range and its own L2 sees the reuse) and then in
// groups of `group_m` row tiles (grouped launches: group by group).
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "sgmv.hpp"

namespace lora {

enum { EPI_BF16 = 0, EPI_LSE = 1, EPI_GRAD = 2 };

struct GemmEpi {
  uint16_t* C;            // EPI_BF16 / EPI_GRAD output
  int64_t ldc;
  // Row maps (nullable = identity): position m reads A row a_rows[m] and
  // writes C row c_rows[m] (the LoRA vector row too); rowscale[m] multiplies
  // the base product of row m before the LoRA slab is added.
  const int32_t* a_rows;
  const int32_t* c_rows;
  const float* rowscale;
  // Grouped rows (g_tile non-null): positions form n_groups consecutive groups,
  // group g spanning [g_off[g*g_stride], g_off[(g+1)*g_stride]) and multiplying
  // its own B at B + g*ldb_group; g_tile[g] = first 256-row tile of group g.
  const int32_t* g_tile;
  const int32_t* g_off;
  int g_stride;
  int n_groups;
  int64_t ldb_group;
  // EPI_BF16 with the LoRA expand fused (nullable vec = plain GEMM): for the
  // row at segment position m, owned by adapter a, add s_a * vec[tok] . M_a^T
  // with M_a [N][r_a] = B_a at b_off of the pack lmat (use_b_off = 1), or
  // M_a = A_a^T read in place from A_a [r_a][lmat_ld] at a_off (use_b_off = 0).
  const uint16_t* vec;    // scaled vector, bf16 hi plane [rows][vec_ld]: row = the C row
                          // (c_rows[m]), or the position m itself with vec_by_pos
  int64_t vec_plane;      // lo plane at vec + vec_plane
  int vec_ld;
  int vec_by_pos;
  int use_b_off;
  int64_t lmat_ld;
  const uint16_t* lmat;
  const lora_adapter_desc* desc;
  // A second weight operand B2 (same ldb and group stride as B), for
  //   k_split > 0 (K split, a multiple of 64): k >= k_split reads B2 at
  //     column k - k_split, and both LoRA sets (vec/lmat/desc and
  //     vec2/lmat2/desc2) are added to every row;
  //   glu = 1 (below).
  const uint16_t* B2;
  int64_t c_off2;
  int k_split;
  const uint16_t* vec2;
  const uint16_t* lmat2;
  const lora_adapter_desc* desc2;
  // SwiGLU fused into the epilogue (EPI_BF16):
  //   glu = 1: a 256-column tile holds 128 columns n0.. of the first product
  //     (B, LoRA set 1) and the same 128 columns of the second (B2, set 2);
  //     C gets [gate | up] rows (up at column c_off2) and hout[row][n] =
  //     silu(gate) * up from the stored bf16 values;
  //   glu = 2: the product is dh (C nullable: stored only when given); with
  //     gu rows [gate | up] (stride ld_gu, up at c_off2) the epilogue writes
  //     dgu rows [dgate | dup] (stride ld_dgu, dup at c_off2).
  int glu;
  uint16_t* hout;
  int64_t ld_h;
  const uint16_t* gu;
  int64_t ld_gu;
  uint16_t* dgu;
  int64_t ld_dgu;
  const uint8_t* active;
  const int32_t* adpos;   // [M] adapter of each row position, -1 for rows without one
  int n_ad;
  float* part_m;          // EPI_LSE: [tiles_n][M]
  float* part_s;          // EPI_LSE: [tiles_n][M]
  float* zt;              // EPI_LSE: [M] target logit
  const int32_t* targets; // EPI_LSE / EPI_GRAD: [M]
  const float* lse;       // EPI_GRAD: [M]
  const float* dlogp;     // EPI_GRAD: [M]
};

constexpr int GBM = 256, GBN = 256;
constexpr float kLog2e = 1.4426950408889634f;


// Operand movement: gfx950 LDS-DMA (global_load_lds_dwordx4) into two LDS
// stages of BK = 64 (each stage: A and B tiles of 256 rows x 128 B = 32 KB),
// double-buffered: step k computes on stage k % 2 while the DMA fills the
// other with k + 1.  A 64-wide k slice is one whole 128-byte line per row, so
// each DMA instruction moves 8 full lines (16 half lines with 32-wide slices
// cost the texture path twice the requests per byte).  The DMA is issued from
// inline assembly with explicit vmcnt waits: the compiler's own counter
// bookkeeping for LDS-DMA would force a full wait before every LDS read (it
// cannot tell which stage a DMA writes).  Rows past the matrix edge are
// clamped to the last row: they only feed output rows or columns that are
// never stored.
constexpr int SBK = 64;                    // k per stage
constexpr int S_CH = SBK / 8;              // 16-byte chunks per LDS row (8)
constexpr int S_TILE = 256 * S_CH;         // uint4 per operand tile per stage (32 KB)
constexpr int NSTAGE = 2;
constexpr int WN = 64;                     // output columns per wave
constexpr int NJ = WN / 32;                // 32-column MFMA tiles per wave
constexpr int NWN = GBN / WN;              // waves along N
constexpr int NWAVES = 2 * NWN;            // waves: two along M, 128 rows each
constexpr int GTHREADS = 64 * NWAVES;
constexpr int DMA_PER_OP = GBM / (8 * NWAVES);   // DMA instructions (8 rows each) per wave,
                                                 // operand and stage

// After the k loop (and a barrier) the operand stages hold the epilogue's
// scratch: the staged output tile, the per-wave LoRA slab tiles and the row
// map (or the logsumexp partials).
constexpr int EPI_SLAB = GBM * 512;                        // bytes: after the staged tile
constexpr int SLAB_LD = WN + 8;                            // bf16 per LDS row of a slab tile
constexpr int SLAB_BYTES = 16 * SLAB_LD * 2;               // per wave
constexpr int EPI_ROW = EPI_SLAB + NWAVES * SLAB_BYTES;
constexpr int RING_BYTES = 2 * NSTAGE * S_TILE * 16;
constexpr int LDS_BYTES = RING_BYTES > EPI_ROW + GBM * 4 ? RING_BYTES : EPI_ROW + GBM * 4;
static_assert(EPI_SLAB + NWN * GBM * 8 <= LDS_BYTES, "logsumexp partials exceed the LDS block");
__shared__ uint4 g_stage[LDS_BYTES / 16];   // [A stages][B stages], then epilogue scratch

__device__ __forceinline__ uint32_t lds_addr(const uint4* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// One 16-byte LDS-DMA per lane: global (base + voff) -> LDS (m0v + 16 * lane).
// base is wave-uniform (SGPR pair), voff a per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16s(uint32_t voff, const void* base, uint32_t m0v) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0v), "v"(voff), "s"(base)
               : "memory");
}

// Fused LoRA expand: for every adapter a owning rows of this wave's 128 rows
// (rows are segment positions, so they span one adapter or a few), add
// (s_a u_tok) . M_a^T to the accumulators as an extra MFMA K-slab of depth r_a.
// The scaled vector is stored as bf16 hi and lo planes, one MFMA each, so the
// slab keeps ~16 significant bits; M_a is bf16-exact.  tok[i] / ad[i] are the
// token and adapter (-1: none) of this lane's fragment rows, loaded before
// the k loop.  An adapter's MFMAs run only for the 32-row tiles holding rows
// of it (a wave spanning two adapters pays for each about once, not twice).
// With M_a = A_a^T (use_b_off = 0) the factor block of a 16-rank slice (16
// rows of A_a x the wave's WN columns) is loaded row-wise into the wave's LDS
// tile `slab` (rows padded by 16 bytes: the transposing reads of 4 rows hit
// distinct banks) and read back transposed, 8 consecutive ranks of one column
// per lane.
__device__ __forceinline__ void lora_slab(const GemmEpi& ep, const uint16_t* vec,
                                          const uint16_t* lmat, const lora_adapter_desc* desc,
                                          int n0, int N, int wn, int lane, uint4* slab,
                                          const int (&vrow)[4], const int (&ad)[4],
                                          f32x16 (&acc)[4][NJ]) {
  const int m_l = lane & 31;
  const int half = lane >> 5;
  int lo = INT32_MAX, hi = -1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (ad[i] >= 0) lo = min(lo, ad[i]), hi = max(hi, ad[i]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    lo = min(lo, __shfl_xor(lo, o));
    hi = max(hi, __shfl_xor(hi, o));
  }
  const int a0 = __builtin_amdgcn_readfirstlane(lo), a1 = __builtin_amdgcn_readfirstlane(hi);
  for (int a = a0; a <= a1; ++a) {
    bool tile_has[4], mine = false;   // wave-uniform: 32-row tiles holding rows of a
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile_has[i] = __any(ad[i] == a);
      mine |= tile_has[i];
    }
    if (!mine) continue;                            // adapter absent from this wave's rows
    const lora_adapter_desc d = desc[a];
    const int r = d.rank;
    const uint16_t* mat = lmat + (ep.use_b_off ? d.b_off : d.a_off);
    for (int sl = 0; sl * 16 < r; ++sl) {
      const int c = sl * 16 + 8 * half;
      const bool cok = c < r;
      uint4 h[4], l[4], v[NJ];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = l[i] = make_uint4(0, 0, 0, 0);
        if (ad[i] == a && cok) {
          const uint16_t* vp = vec + (int64_t)vrow[i] * ep.vec_ld + c;
          h[i] = *(const uint4*)vp;
          l[i] = *(const uint4*)(vp + ep.vec_plane);
        }
      }
      if (ep.use_b_off) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int n = n0 + wn * WN + j * 32 + m_l;
          v[j] = make_uint4(0, 0, 0, 0);
          if (n < N && cok) v[j] = *(const uint4*)(mat + (int64_t)n * r + c);
        }
      } else {
        // rows sl*16 .. +15 of A_a (zero past rank r), columns nw .. nw + WN - 1
        // (zero past N), 16 bytes per lane and load
        const int nw = n0 + wn * WN;
#pragma unroll
        for (int t = 0; t < NJ; ++t) {
          const int q = lane + 64 * t;
          const int row = q / (WN / 8), cc = q % (WN / 8);
          uint4 val = make_uint4(0, 0, 0, 0);
          if (sl * 16 + row < r && nw + cc * 8 < N)
            val = *(const uint4*)(mat + (int64_t)(sl * 16 + row) * ep.lmat_ld + nw + cc * 8);
          slab[row * (SLAB_LD / 8) + cc] = val;
        }
        // lane: column j*32 + m_l, ranks 8*half + 0..3 and 4..7 of the slice
        const int q = (lane >> 2) & 3, jj = lane & 3;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int col = j * 32 + 16 * ((lane >> 4) & 1) + 4 * jj;
          const uint32_t off = (uint32_t)(((8 * half + q) * SLAB_LD + col) * 2);
          const uint2 lo4 = tr_read(slab, off);
          const uint2 hi4 = tr_read(slab, off + 4 * SLAB_LD * 2);
          v[j] = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!tile_has[i]) continue;   // no row of adapter a in this 32-row tile
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[i][j] = mfma32(as_bf16x8(v[j]), as_bf16x8(h[i]), acc[i][j]);
          acc[i][j] = mfma32(as_bf16x8(v[j]), as_bf16x8(l[i]), acc[i][j]);
        }
      }
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(GTHREADS, 1) void gemm_nt_kernel(const uint16_t* __restrict__ A,
                                                         const uint16_t* __restrict__ B, int M,
                                                         int N, int K, int64_t lda, int64_t ldb,
                                                         GemmEpi ep, int tiles_m, int tiles_n,
                                                         int group_m) {
  // ---- tile id: XCD-contiguous, then grouped along M.  Grouped launches are
  // sized for a bound on the row tiles; the live count comes from the device
  // prefix, and the live tiles are split evenly over the XCDs (the surplus
  // blocks of every XCD exit), so no XCD is left with only dead tiles.
  const int live_m = ep.g_tile ? ep.g_tile[ep.n_groups] : tiles_m;   // <= tiles_m
  const int num = live_m * tiles_n;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, loc = bid >> 3;
  const int per = num >> 3, rem = num & 7;
  if (loc >= per + (xcd < rem ? 1 : 0)) return;
  const int t = (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
  int tm, tn, g = 0;
  if (ep.g_tile) {
    // grouped: tiles run group by group (group g owns tiles g_tile[g] * tiles_n
    // .. g_tile[g + 1] * tiles_n), row tiles fastest; a group of more than
    // 2 group_m row tiles runs in blocks of group_m row tiles.  The tiles one
    // XCD runs at a time then share their group's weight panels and row
    // panels in its L2
    g = find_bucket(ep.g_tile, ep.n_groups + 1, t / tiles_n);
    const int nr = ep.g_tile[g + 1] - ep.g_tile[g];
    const int bm = nr <= 2 * group_m ? nr : group_m;
    const int in = t - ep.g_tile[g] * tiles_n;
    const int blk = in / (bm * tiles_n);
    const int first = blk * bm;
    const int gm = min(nr - first, bm);
    const int r = in - blk * bm * tiles_n;
    tm = first + r % gm;   // row tile within the group
    tn = r / gm;
  } else {
    const int gsz = group_m * tiles_n;
    const int grp = t / gsz;
    const int first_m = grp * group_m;
    const int gm = min(live_m - first_m, group_m);
    const int in = t - grp * gsz;
    tm = first_m + in % gm;
    tn = in / gm;
  }
  const bool glu1 = EPI == EPI_BF16 && ep.glu == 1;   // [gate | up] halves in one tile
  int m0 = tm * GBM;
  const int n0 = tn * (glu1 ? GBN / 2 : GBN);
  int Mlim = M;   // positions >= Mlim are past this tile's row range
  const uint16_t* B2g = ep.B2;   // second operand of this tile's group (K split, glu)
  if (ep.g_tile) {
    m0 = ep.g_off[g * ep.g_stride] + tm * GBM;
    Mlim = ep.g_off[(g + 1) * ep.g_stride];
    B += (int64_t)g * ep.ldb_group;
    if (ep.B2) B2g = ep.B2 + (int64_t)g * ep.ldb_group;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;

  // acc[i][j] holds the transposed 32x32 sub-tile: register g of lane l is
  // C[m = wm*128 + i*32 + l%32][n = wn*64 + j*32 + 8*(g/4) + 4*(l/32) + g%4],
  // so each lane owns runs of 4 consecutive output columns.
  f32x16 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 16; ++g) acc[i][j][g] = 0.f;

  // epilogue row metadata, loaded now so its latency hides under the k loop
  const int m_l = lane & 31;
  const int n_q = 4 * (lane >> 5);
  int tok[4], ad[4];
  float rs[4];
  int gy[4];          // EPI_LSE / EPI_GRAD: target; EPI_GRAD: dlogp, lse of the rows
  float gd[4], gl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm * 128 + i * 32 + m_l;
    tok[i] = row < Mlim ? (ep.c_rows ? ep.c_rows[row] : row) : -1;
    ad[i] = (EPI == EPI_BF16 && ep.vec && row < Mlim) ? ep.adpos[row] : -1;
    rs[i] = (EPI == EPI_BF16 && ep.rowscale && row < Mlim) ? ep.rowscale[row] : 1.f;
    gy[i] = -1;
    gd[i] = 0.f;
    gl[i] = 0.f;
    if (EPI == EPI_LSE && row < M) gy[i] = ep.targets[row];
    if (EPI == EPI_GRAD && row < M) {
      gy[i] = ep.targets[row];
      gd[i] = ep.dlogp[row];
      gl[i] = ep.lse[row];
      if (gy[i] < 0 || gy[i] >= N) gd[i] = 0.f;   // invalid target: zero row
    }
  }

  const int KT = K / SBK;
  uint4* sA = g_stage;
  uint4* sB = g_stage + NSTAGE * S_TILE;

  // This lane's DMA sources as 32-bit byte offsets from a wave-uniform base
  // (the SGPR-addressed form of the DMA: stepping k costs one scalar add and
  // no vector work).  A rows gathered through perm are offsets from A itself
  // (the host checks they fit in 32 bits); other rows are offsets from the
  // tile's first row.  Rows past the edge are clamped to the last row: they
  // only feed outputs that are never stored.
  // Instruction i of wave w fills rows 8 (w DMA_PER_OP + i) .. + 7 of a
  // stage: lane L lands in row L / 8, physical chunk L % 8, i.e. logical
  // chunk (L % 8) ^ lds_sw(row).
  uint32_t offA[DMA_PER_OP], offB[DMA_PER_OP];
  const uint16_t* baseA = ep.a_rows ? A : A + (int64_t)m0 * lda;
  // glu: the waves loading tile rows 128.. load the second product's rows
  const bool bhalf = glu1 && wave >= NWAVES / 2;
  const uint16_t* baseB = (bhalf ? B2g : B) + (int64_t)n0 * ldb;
  // K split: k >= ksplit reads the second operand (same row offsets)
  const int ksplit = ep.k_split > 0 ? ep.k_split : K;
  const uint16_t* baseB2 = ep.k_split > 0 ? B2g + (int64_t)n0 * ldb : baseB;
  auto bsrc = [&](int k0) { return k0 < ksplit ? baseB + k0 : baseB2 + (k0 - ksplit); };
#pragma unroll
  for (int i = 0; i < DMA_PER_OP; ++i) {
    const int row = (wave * DMA_PER_OP + i) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ lds_sw(row);
    const int ra = min(m0 + row, Mlim - 1);
    const int rb = min(n0 + (glu1 ? (row & (GBN / 2 - 1)) : row), N - 1);
    const int64_t oa = ep.a_rows ? (int64_t)ep.a_rows[ra] * lda : (int64_t)(ra - m0) * lda;
    offA[i] = (uint32_t)((oa + chunk * 8) * 2);
    offB[i] = (uint32_t)(((int64_t)(rb - n0) * ldb + chunk * 8) * 2);
  }
  const uint32_t ldsA = __builtin_amdgcn_readfirstlane(lds_addr(sA + wave * DMA_PER_OP * 8 * S_CH));
  const uint32_t ldsB = __builtin_amdgcn_readfirstlane(lds_addr(sB + wave * DMA_PER_OP * 8 * S_CH));
  // DMA of operand rows (instruction i of this wave) for k0 into stage st
  auto dmaA = [&](int st, int i, const uint16_t* kb) {
    dma16s(offA[i], kb, ldsA + (uint32_t)(st * S_TILE + i * 64) * 16u);
  };
  auto dmaB = [&](int st, int i, const uint16_t* kb) {
    dma16s(offB[i], kb, ldsB + (uint32_t)(st * S_TILE + i * 64) * 16u);
  };

  // prologue: stages 0 and 1 both in flight (every block starts at once, so
  // the first loads queue behind the whole chip's); stage 0 landed and
  // visible to every wave.  Step 0 issues no DMA: its barrier waits for
  // stage 1.
  static_assert(2 * DMA_PER_OP == 8, "the prologue wait counts one stage of DMA");
#pragma unroll
  for (int i = 0; i < DMA_PER_OP; ++i) dmaA(0, i, baseA);
#pragma unroll
  for (int i = 0; i < DMA_PER_OP; ++i) dmaB(0, i, bsrc(0));
  if (KT > 1) {
#pragma unroll
    for (int i = 0; i < DMA_PER_OP; ++i) dmaA(1, i, baseA + SBK);
#pragma unroll
    for (int i = 0; i < DMA_PER_OP; ++i) dmaB(1, i, bsrc(SBK));
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }

  const int frag_row = lane & 31;   // row within a 32-row MFMA tile
  const int frag_half = lane >> 5;  // which 8-wide k half of a 16-wide k slice
  const int sw = lds_sw(frag_row);  // swizzle of every fragment row of this lane
  int a_row[4], b_row[NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i) a_row[i] = (wm * 128 + i * 32 + frag_row) * S_CH;
#pragma unroll
  for (int j = 0; j < NJ; ++j) b_row[j] = (wn * WN + j * 32 + frag_row) * S_CH;
  int cq[4];   // physical chunk of this lane's fragment in 16-wide slice q
#pragma unroll
  for (int q = 0; q < 4; ++q) cq[q] = (2 * q + frag_half) ^ sw;

  bf16x8 fa[2][4], fb[2][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[0][i] = as_bf16x8(sA[a_row[i] + cq[0]]);
#pragma unroll
  for (int j = 0; j < NJ; ++j) fb[0][j] = as_bf16x8(sB[b_row[j] + cq[0]]);

  // One k step (64 k, 4 slices of 16) on stage S (static, so every LDS
  // address is base + immediate).  Each slice is a phase of 4 NJ groups of
  // one MFMA; the LDS fragment reads for the next slice go into the first
  // groups, and the step's 2 DMA_PER_OP DMA instructions (the other stage, k
  // step kt + 1) one per group of the first phase, so the vector-memory, LDS
  // and scalar work issues in the shadow of the matrix pipe and the DMA has
  // most of the step to land.  The step's one barrier sits in the middle of
  // its last phase, whose second half reads the next stage's first slice
  // under the remaining MFMAs.  sched_barrier keeps the groups
  // in this order.  After the wait and the barrier the next stage is visible
  // and its first slice is read.
  auto step = [&](auto S_, int kt) {
    constexpr int S = decltype(S_)::value;
    constexpr int SN = 1 - S;
    const uint4* At = sA + S * S_TILE;
    const uint4* Bt = sB + S * S_TILE;
    const uint4* An = sA + SN * S_TILE;
    const uint4* Bn = sB + SN * S_TILE;
    const bool more = kt >= 1 && kt + 1 < KT;   // step 1 came with the prologue
    const int k0 = (more ? kt + 1 : kt) * SBK;
    const uint16_t* ka = baseA + k0;
    const uint16_t* kb = bsrc(k0);
    constexpr int G = 4 * NJ;   // MFMA groups per phase
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cur = q & 1, nxt = cur ^ 1;
      static_assert(G == 2 * DMA_PER_OP, "one DMA per group of the first phase");
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int i = g / NJ, j = g % NJ;
        if (q == 3 && g == G / 2) {
          // this wave's reads of stage S are complete and its DMA of stage SN
          // has landed; after the barrier both hold for every wave, so the
          // rest of the phase reads the next stage's first slice and the next
          // step may refill stage S
          asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
        acc[i][j] = mfma32(fb[cur][j], fa[cur][i], acc[i][j]);
        if (q < 3) {
          if (g < 4) fa[nxt][g] = as_bf16x8(At[a_row[g] + cq[q + 1]]);
          else if (g < 4 + NJ) fb[nxt][g - 4] = as_bf16x8(Bt[b_row[g - 4] + cq[q + 1]]);
        } else if (g >= G / 2) {
          // 4 + NJ reads over the last G / 2 groups
#pragma unroll
          for (int t = 0; t < 4 + NJ; ++t) {
            if (t * (G / 2) / (4 + NJ) != g - G / 2) continue;
            if (t < 4) fa[nxt][t] = as_bf16x8(An[a_row[t] + cq[0]]);
            else fb[nxt][t - 4] = as_bf16x8(Bn[b_row[t - 4] + cq[0]]);
          }
        }
        if (q == 0 && more) {   // the whole next stage as early as possible
          if (g < DMA_PER_OP) dmaA(SN, g, ka);
          else dmaB(SN, g - DMA_PER_OP, kb);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // A wave whose 128 rows all lie past the tile's row range (the tail tile of
  // a group or of the matrix) keeps the other waves' DMA and barrier cadence
  // but skips the fragment reads and MFMAs.
  const bool live = m0 + wm * 128 < Mlim;
  int kt = 0;
  if (live) {
    for (; kt + 2 <= KT; kt += 2) {
      step(std::integral_constant<int, 0>{}, kt);
      step(std::integral_constant<int, 1>{}, kt + 1);
    }
    if (kt < KT) step(std::integral_constant<int, 0>{}, kt);
  } else {
    for (; kt < KT; ++kt) {
      if (kt >= 1 && kt + 1 < KT) {
        const int k0 = (kt + 1) * SBK;
        const int sn = (kt + 1) & 1;
#pragma unroll
        for (int i = 0; i < DMA_PER_OP; ++i) dmaA(sn, i, baseA + k0);
#pragma unroll
        for (int i = 0; i < DMA_PER_OP; ++i) dmaB(sn, i, bsrc(k0));
      }
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA may outlive the block

  // ---- epilogues

  // Output tiles are staged in the idle ring (256 rows x 512 B, 16-byte chunks
  // swizzled by row) and written as whole 512-byte rows, 2 rows per wave store.
  // s_row holds each staged row's destination (-1: not stored).
  char* T = (char*)g_stage;
  int* s_row = (int*)(T + EPI_ROW);
  // glu = 1: staged columns 0..127 are the first product, 128..255 the second
  auto stage_rows = [&]() {
    if (wn == 0 && lane < 32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s_row[wm * 128 + i * 32 + lane] = tok[i];
    }
  };
  auto stage = [&](int i, int j, int q, uint2 v) {
    const int row = wm * 128 + i * 32 + m_l;
    const int chunk = wn * (WN / 8) + j * 4 + q;
    *(uint2*)(T + row * 512 + ((chunk ^ (row & 31)) << 4) + ((lane >> 5) << 3)) = v;
  };
  auto staged = [&](int row, int c) {
    return *(const uint4*)(T + row * 512 + ((c ^ (row & 31)) << 4));
  };
  constexpr int NIT = GBM / NWAVES / 2;   // store iterations per wave (2 rows each)
  auto store_rows = [&]() {
    const int c = lane & 31;
    if (EPI == EPI_BF16 && ep.glu == 2) {
      // the saved [gate | up] values of every row this lane stores, loaded
      // up front (the accumulators are dead by now) so their latency is paid
      // once
      uint4 gq[NIT], uq[NIT];
#pragma unroll
      for (int k = 0; k < NIT; ++k) {
        const int row = wave * (GBM / NWAVES) + 2 * k + (lane >> 5);
        const int crow = s_row[row];
        const int col = n0 + c * 8;
        gq[k] = uq[k] = make_uint4(0, 0, 0, 0);
        if (crow >= 0 && col < N) {
          const uint16_t* gp = ep.gu + (int64_t)crow * ep.ld_gu + col;
          gq[k] = *(const uint4*)gp;
          uq[k] = *(const uint4*)(gp + ep.c_off2);
        }
      }
#pragma unroll
      for (int k = 0; k < NIT; ++k) {
        const int row = wave * (GBM / NWAVES) + 2 * k + (lane >> 5);
        const int crow = s_row[row];
        const int col = n0 + c * 8;
        if (crow >= 0 && col < N) {
          const uint4 v = staged(row, c);
          if (ep.C) *(uint4*)(ep.C + (int64_t)crow * ep.ldc + col) = v;
          uint4 dg, du;
          swiglu_bwd8(v, gq[k], uq[k], dg, du);
          uint16_t* dp = ep.dgu + (int64_t)crow * ep.ld_dgu + col;
          *(uint4*)dp = dg;
          *(uint4*)(dp + ep.c_off2) = du;
        }
      }
      return;
    }
#pragma unroll 4
    for (int k = 0; k < NIT; ++k) {
      const int row = wave * (GBM / NWAVES) + 2 * k + (lane >> 5);
      const int crow = s_row[row];
      const uint4 v = staged(row, c);
      if (EPI == EPI_BF16 && ep.glu == 1) {
        const int part = c >> 4;   // 0: gate, 1: up
        const int col = n0 + (c & 15) * 8;
        if (crow >= 0 && col < N) {
          *(uint4*)(ep.C + (int64_t)crow * ep.ldc + part * ep.c_off2 + col) = v;
          // h: every lane takes 4 columns, (c & 15) * 8 + 4 * part ..
          const char* gp = T + row * 512 + (((c & 15) ^ (row & 31)) << 4) + part * 8;
          const char* up = T + row * 512 + ((((c & 15) + 16) ^ (row & 31)) << 4) + part * 8;
          const uint2 g4 = *(const uint2*)gp, u4 = *(const uint2*)up;
          const uint2 h4 = make_uint2(
              pk16(swiglu_fwd1(lo16(g4.x), lo16(u4.x)), swiglu_fwd1(hi16(g4.x), hi16(u4.x))),
              pk16(swiglu_fwd1(lo16(g4.y), lo16(u4.y)), swiglu_fwd1(hi16(g4.y), hi16(u4.y))));
          *(uint2*)(ep.hout + (int64_t)crow * ep.ld_h + col + 4 * part) = h4;
        }
      } else {
        const int col = n0 + c * 8;
        if (crow >= 0 && col < N) *(uint4*)(ep.C + (int64_t)crow * ep.ldc + col) = v;
      }
    }
  };

  if constexpr (EPI == EPI_BF16) {
    if (ep.rowscale) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int g = 0; g < 16; ++g) acc[i][j][g] *= rs[i];
    }
    __syncthreads();   // every wave is done reading the ring
    if (ep.vec) {
      // one expand (set 2 for the second half of a glu tile), or both sets
      // for a K split; a loop, so the slab is instantiated once
      const int sets = (ep.k_split > 0 && ep.vec2) ? 2 : 1;
      const bool upper = glu1 && wn >= NWN / 2;
      const int wn_eff = glu1 ? wn % (NWN / 2) : wn;   // column slice within its product
      uint4* slab = (uint4*)(T + EPI_SLAB + wave * SLAB_BYTES);
      int vrow[4];   // vector row of each fragment row: its C row, or its position
#pragma unroll
      for (int i = 0; i < 4; ++i) vrow[i] = ep.vec_by_pos ? m0 + wm * 128 + i * 32 + m_l : tok[i];
#pragma unroll 1
      for (int set = 0; set < sets; ++set) {
        const bool two = upper || set == 1;
        lora_slab(ep, two ? ep.vec2 : ep.vec, two ? ep.lmat2 : ep.lmat, two ? ep.desc2 : ep.desc,
                  n0, N, wn_eff, lane, slab, vrow, ad, acc);
      }
    }
    stage_rows();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          stage(i, j, q, make_uint2(pack2bf(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                    pack2bf(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])));
    __syncthreads();
    store_rows();
  } else if constexpr (EPI == EPI_LSE) {
    // (max, sum) pairs of the NWN column slices of the waves, then merged per
    // row in slice order (deterministic)
    __syncthreads();   // every wave is done reading the ring
    float2 (*red_s)[GBM] = (float2 (*)[GBM])(T + EPI_SLAB);
    const int cbase = n0 + wn * WN;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = wm * 128 + i * 32 + m_l;
      const int row = m0 + rl;
      // this lane's 32 values of row `row`: columns cbase + j*32 + 8q + n_q + e
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (cbase + j * 32 + 8 * q + n_q + e < N) mx = fmaxf(mx, acc[i][j][4 * q + e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float sm = 0.f;
      if (mx != -INFINITY) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (cbase + j * 32 + 8 * q + n_q + e < N)
                sm += exp2f((acc[i][j][4 * q + e] - mx) * kLog2e);
      }
      sm += __shfl_xor(sm, 32);
      if (row < M) {
        const int yo = gy[i] - cbase;
        // column offset yo = j*32 + 8q + n_q + e
        if (yo >= 0 && yo < WN && cbase + yo < N && ((yo >> 2) & 1) == (lane >> 5)) {
          const int jj = yo >> 5, qq = (yo >> 3) & 3, ee = yo & 3;
          float zv = 0.f;
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (j == jj && q == qq && e == ee) zv = acc[i][j][4 * q + e];
          ep.zt[row] = zv;
        }
      }
      if (lane < 32) red_s[wn][rl] = make_float2(mx, sm);
    }
    __syncthreads();
    for (int r = tid; r < GBM; r += GTHREADS) {
      if (m0 + r >= M) continue;
      float mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < NWN; ++w) mx = fmaxf(mx, red_s[w][r].x);
      float sm = 0.f;
#pragma unroll
      for (int w = 0; w < NWN; ++w)
        if (red_s[w][r].x != -INFINITY) sm += red_s[w][r].y * exp2f((red_s[w][r].x - mx) * kLog2e);
      ep.part_m[(int64_t)tn * M + m0 + r] = mx;
      ep.part_s[(int64_t)tn * M + m0 + r] = sm;
    }
  } else {  // EPI_GRAD: G = d (onehot(y) - exp(z - lse)), staged and stored like EPI_BF16
    __syncthreads();
    stage_rows();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * WN + j * 32 + 8 * q + n_q;
          float gv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pr = exp2f((acc[i][j][4 * q + e] - gl[i]) * kLog2e);
            gv[e] = gd[i] == 0.f ? 0.f : gd[i] * ((col + e == gy[i] ? 1.f : 0.f) - pr);
          }
          stage(i, j, q, make_uint2(pack2bf(gv[0], gv[1]), pack2bf(gv[2], gv[3])));
        }
    __syncthreads();
    store_rows();
  }
}

}  // namespace lora

namespace lora_host {

using namespace lora;

static int pick_group_m(int tiles_m) { return tiles_m < 4 ? tiles_m : 4; }

template <int EPI>
static lora_status launch_gemm(const uint16_t* A, const uint16_t* B, int M, int N, int K,
                               int64_t lda, int64_t ldb, const GemmEpi& ep, hipStream_t s,
                               int group_m, int64_t a_rows_bound = 0, int tiles_m_bound = 0) {
  if (M <= 0 || N <= 0) return LORA_OK;
  if (ep.a_rows && (int64_t)a_rows_bound * lda * 2 >= ((int64_t)1 << 32)) {
    set_error("gemm: gathered operand of %lld bytes exceeds the 4 GiB the row offsets address",
              (long long)(a_rows_bound * lda * 2));
    return LORA_E_UNSUPPORTED;
  }
  const int tiles_m = ep.g_tile ? tiles_m_bound : (int)cdiv(M, GBM);
  const int tiles_n = (int)cdiv(N, EPI == EPI_BF16 && ep.glu == 1 ? GBN / 2 : GBN);
  if (EPI == EPI_BF16 && ep.glu == 1 && (!ep.B2 || !ep.hout || ep.k_split > 0)) {
    set_error("gemm: glu needs B2 and hout, and no K split");
    return LORA_E_INVALID_ARG;
  }
  if (EPI == EPI_BF16 && ep.glu == 2 && (!ep.gu || !ep.dgu || ep.vec2)) {
    set_error("gemm: glu backward needs gu and dgu, one LoRA set");
    return LORA_E_INVALID_ARG;
  }
  if (ep.k_split > 0 && (ep.k_split % SBK || ep.k_split >= K || !ep.B2)) {
    set_error("gemm: K split %d must be a multiple of %d below K = %d, with B2", ep.k_split, SBK, K);
    return LORA_E_INVALID_ARG;
  }
  if (tiles_m <= 0) return LORA_OK;
  if (group_m <= 0) group_m = pick_group_m(tiles_m);
  if (group_m > tiles_m) group_m = tiles_m;
  const size_t lds = 0;  // operand tiles are static LDS objects
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)gemm_nt_kernel<EPI>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr_set = true;
  }
  hipLaunchKernelGGL(gemm_nt_kernel<EPI>, dim3(tiles_m * tiles_n), dim3(GTHREADS), lds, s, A, B, M, N,
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

lora_status gemm_nt_rows(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                         int64_t lda, int64_t ldb, int64_t ldc, const GemmRows& f, hipStream_t s,
                         int group_m) {
  GemmEpi ep{};
  ep.C = C;
  ep.ldc = ldc;
  ep.a_rows = f.a_rows;
  ep.c_rows = f.c_rows;
  ep.rowscale = f.rowscale;
  ep.g_tile = f.g_tile;
  ep.g_off = f.g_off;
  ep.g_stride = f.g_stride;
  ep.n_groups = f.n_groups;
  ep.ldb_group = f.ldb_group;
  ep.vec = f.vec;
  ep.vec_plane = f.vec_plane;
  ep.vec_ld = f.vec_ld;
  ep.vec_by_pos = f.vec_by_pos;
  ep.use_b_off = f.use_b_off;
  ep.lmat_ld = f.lmat_ld;
  ep.lmat = f.lmat;
  ep.desc = f.desc;
  ep.B2 = f.B2;
  ep.c_off2 = f.c_off2;
  ep.k_split = f.k_split;
  ep.vec2 = f.vec2;
  ep.lmat2 = f.lmat2;
  ep.desc2 = f.desc2;
  ep.glu = f.glu;
  ep.hout = f.hout;
  ep.ld_h = f.ld_h;
  ep.gu = f.gu;
  ep.ld_gu = f.ld_gu;
  ep.dgu = f.dgu;
  ep.ld_dgu = f.ld_dgu;
  ep.adpos = f.adpos;
  ep.n_ad = f.n_ad;
  return launch_gemm<EPI_BF16>(A, B, M, N, K, lda, ldb, ep, s, group_m, f.a_rows_bound,
                               f.tiles_m_bound);
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
