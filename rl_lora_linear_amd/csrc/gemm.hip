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
// scratch: first the staged LoRA expand operands (below), then the staged
// output tile and the row map (or the logsumexp partials).
constexpr int EPI_SLAB = GBM * 512;                        // bytes: after the staged tile
constexpr int EPI_ROW = EPI_SLAB;
constexpr int RING_BYTES = 2 * NSTAGE * S_TILE * 16;
// LoRA expand staging: the tile's scaled vector rows (hi and lo planes, 256
// rows x 64 ranks each, 16-byte chunks swizzled by row like the operand
// stages), then the factor blocks of one batch of runs, then the row and run
// tables.
constexpr int X_LDS = 160 * 1024;
constexpr int XV_PLANE = GBM * 128;                        // bytes per vector plane
constexpr int XM_OFF = 2 * XV_PLANE;                       // factor blocks
constexpr int X_TAB_OFF = X_LDS - 11 * 1024;               // tables (11 KB)
constexpr int XM_CHUNKS = (X_TAB_OFF - XM_OFF) / 1024 * 64;   // 16-byte chunks, whole DMA rounds
constexpr int LDS_BYTES = X_LDS;
static_assert(RING_BYTES <= LDS_BYTES && EPI_ROW + GBM * 4 <= LDS_BYTES, "LDS block too small");
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

// One 16-byte LDS-DMA per lane from a per-lane 64-bit address:
// global g -> LDS (m0v + 16 * lane).
__device__ __forceinline__ void dma16v(const void* g, uint32_t m0v) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0v), "v"(g) : "memory");
}

// 16-byte chunks of one run's staged factor block: B_a rows n0.. (cols rows of
// r ranks), or A_a's r rows over cols columns plus one pad chunk per row (the
// transposing reads of 4 rows then hit distinct banks).
__device__ __forceinline__ int xm_chunks(int r, int cols, int use_b_off) {
  return use_b_off ? cols * (r >> 3) : r * (cols / 8 + 1);
}

// Fused LoRA expand, staged through LDS.  Every row m of the tile owned by
// adapter a gets (s_a u_m) . M_a^T added to its accumulators: one extra MFMA
// K-slab of depth r_a per plane (the scaled vector is stored as bf16 hi and lo
// planes, so the slab keeps ~16 significant bits; M_a is bf16-exact).  With
// M_a = B_a (use_b_off = 1) a staged row is one column's r_a ranks; with M_a =
// A_a^T (use_b_off = 0) A_a's rows are staged over the tile's columns and read
// back transposed, 8 consecutive ranks of one column per lane.
//
// Rows come in runs of one adapter (segment order).  Per LoRA set (a pass),
// the tile's vector rows and the factor blocks of a batch of runs move to LDS
// in one round of LDS-DMA, and every wave then runs its MFMAs from LDS: one
// memory round trip per pass and batch, where loading operands per adapter
// and 16-rank slice paid one per slice.  A run's MFMAs run only for the
// 32-row tiles holding rows of it.  glu = 1 tiles run the first set in the
// waves of the first column half and the second set in the others; a K split
// runs both sets over every row.  Called by every thread of the block after
// the k loop, with the ring free; ends with a barrier (LDS free again).
// LDS barrier without a wait on vector memory (DMA of operand stages may be
// in flight): LDS writes before it are visible to every wave after it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Expand tables in the LDS above the operand ring (untouched by the k loop).
struct XTabs {
  int* ad;        // adapter of each row (-1: none)
  int* rid;       // run of each row (-1: none)
  int* vrow;      // vector row of each row
  int* rad;       // adapter of each run
  int* rank;      // [2][runs] rank per set
  int64_t* moff;  // [2][runs] factor offset per set
  int* wc;        // runs started per 64 rows
};
__device__ __forceinline__ XTabs x_tabs(char* X) {
  XTabs t;
  t.ad = (int*)(X + X_TAB_OFF);
  t.rid = t.ad + GBM;
  t.vrow = t.rid + GBM;
  t.rad = t.vrow + GBM;
  t.rank = t.rad + GBM;
  t.moff = (int64_t*)(t.rank + 2 * GBM);
  t.wc = (int*)(t.moff + 2 * GBM);
  return t;
}
static_assert(6 * GBM * 4 + 2 * GBM * 8 + 64 <= X_LDS - X_TAB_OFF, "expand tables");

struct XDesc {
  int rank;
  int64_t moff;
};

__device__ __forceinline__ int x_passes(const GemmEpi& ep, bool glu1) {
  return ((glu1 || ep.k_split > 0) && ep.vec2) ? 2 : 1;
}

// Before the k loop (the row metadata has landed with the first stage): the
// tile's rows in runs of one adapter (a row starts a run when its adapter
// differs from the previous row's), and the run descriptors of both LoRA sets
// loaded into registers, one per thread (passes * runs <= 512), so that they
// land during the k loop.  Returns the number of runs.
__device__ __forceinline__ int expand_prep(const GemmEpi& ep, char* X, int wave, int lane,
                                           bool glu1, const int (&ad)[4], const int (&vrow)[4],
                                           XDesc& dk) {
  const XTabs tb = x_tabs(X);
  const int wm = wave / NWN, wn = wave % NWN;
  if (wn == 0 && lane < 32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + i * 32 + lane;
      tb.ad[row] = ad[i];
      tb.vrow[row] = ad[i] >= 0 ? vrow[i] : 0;   // rows without an adapter read row 0 (unused)
    }
  }
  lds_barrier();
  const int trow = wave * 64 + lane;   // rows 0..255 in waves 0..3
  const int a_t = wave < GBM / 64 ? tb.ad[trow] : -1;
  const int a_p = (wave < GBM / 64 && trow > 0) ? tb.ad[trow - 1] : -1;
  const bool start = a_t >= 0 && a_t != a_p;
  const uint64_t bal = __ballot(start);
  const int incl = __popcll(bal & ((2ull << lane) - 1));
  if (wave < GBM / 64 && lane == 0) tb.wc[wave] = __popcll(bal);
  lds_barrier();
  int n_runs = 0, before = 0;
#pragma unroll
  for (int w = 0; w < GBM / 64; ++w) {
    const int c = tb.wc[w];
    if (w < wave) before += c;
    n_runs += c;
  }
  if (wave < GBM / 64) {
    tb.rid[trow] = a_t >= 0 ? before + incl - 1 : -1;
    if (start) tb.rad[before + incl - 1] = a_t;
  }
  lds_barrier();
  dk.rank = 0;
  dk.moff = 0;
  const int k = threadIdx.x;
  if (k < x_passes(ep, glu1) * n_runs) {
    const int p = k >= n_runs, kk = k - p * n_runs;
    // the field's address is chosen, not its value, so nothing waits on the
    // loads before the expand uses them
    const lora_adapter_desc* d = (p ? ep.desc2 : ep.desc) + tb.rad[kk];
    dk.rank = d->rank;
    dk.moff = *(ep.use_b_off ? &d->b_off : &d->a_off);
  }
  return n_runs;
}

// Each run's rank and factor offset, per set, into the tables above the ring:
// written after the k loop (the descriptor loads of expand_prep have landed)
// and before the barrier that precedes lora_expand, so that the expand issues
// its first DMA round without a barrier of its own.
__device__ __forceinline__ void x_tables(const GemmEpi& ep, bool glu1, char* X, int n_runs,
                                         const XDesc& dk) {
  const XTabs tb = x_tabs(X);
  const int k = threadIdx.x;
  if (k < x_passes(ep, glu1) * n_runs) {
    const int p = k >= n_runs, kk = k - p * n_runs;
    tb.rank[p * GBM + kk] = dk.rank;
    tb.moff[p * GBM + kk] = dk.moff;
  }
}

// Fused LoRA expand, staged through LDS.  Every row m of the tile owned by
// adapter a gets (s_a u_m) . M_a^T added to its accumulators: one extra MFMA
// K-slab of depth r_a per plane (the scaled vector is stored as bf16 hi and lo
// planes, so the slab keeps ~16 significant bits; M_a is bf16-exact).  With
// M_a = B_a (use_b_off = 1) a staged row is one column's r_a ranks; with M_a =
// A_a^T (use_b_off = 0) A_a's rows are staged over the tile's columns and read
// back transposed, 8 consecutive ranks of one column per lane.
//
// Per LoRA set (a pass), the tile's vector rows and the factor blocks of a
// batch of runs move to LDS in one round of LDS-DMA, and every wave then runs
// its MFMAs from LDS: one memory round trip per pass and batch, where loading
// operands per adapter and 16-rank slice paid one per slice.  A run's MFMAs
// run only for the 32-row tiles holding rows of it.  glu = 1 tiles run the
// first set in the waves of the first column half and the second set in the
// others; a K split runs both sets over every row.  Called by every thread of
// the block after the k loop and a barrier, with the ring free and the tables
// of expand_prep and x_tables visible; ends with a barrier (LDS free again).
__device__ __forceinline__ void lora_expand(const GemmEpi& ep, char* X, int n0, int N, int wave,
                                            int lane, bool glu1, int n_runs,
                                            f32x16 (&acc)[4][NJ]) {
  const int wm = wave / NWN, wn = wave % NWN;
  const int m_l = lane & 31, half = lane >> 5;
  const XTabs tb = x_tabs(X);
  const int passes = x_passes(ep, glu1);
  const int cols = glu1 ? GBN / 2 : GBN;
  const int wn_eff = glu1 ? wn % (NWN / 2) : wn;
  const int vch = ep.vec_ld / 8;
  // both planes of a pass's vector rows: row r, logical chunk c at chunk
  // r * 8 + (c ^ (r & 7)) of its plane
  auto dma_vec = [&](const uint16_t* vec) {
#pragma unroll
    for (int pl = 0; pl < 2; ++pl)
#pragma unroll
      for (int i = 0; i < GBM * 8 / 64 / NWAVES; ++i) {
        const int q = (wave * (GBM * 8 / 64 / NWAVES) + i) * 64 + lane;
        const int row = q >> 3;
        int c = (q & 7) ^ (row & 7);
        if (c >= vch) c = 0;   // past the vector width: any chunk of the row (unused)
        const uint16_t* src =
            vec + (pl ? ep.vec_plane : 0) + (int64_t)tb.vrow[row] * ep.vec_ld + c * 8;
        dma16v(src, lds_addr((const uint4*)(X + pl * XV_PLANE + (q - lane) * 16)));
      }
  };
  int rid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) rid[i] = tb.rid[wm * 128 + i * 32 + m_l];

  const uint4* XV = (const uint4*)X;
  const uint4* XL = (const uint4*)(X + XV_PLANE);
  const uint4* XM = (const uint4*)(X + XM_OFF);
#pragma unroll 1
  for (int p = 0; p < passes; ++p) {
    const uint16_t* lmat = p ? ep.lmat2 : ep.lmat;
    const int* rk = tb.rank + p * GBM;
    const int64_t* mo = tb.moff + p * GBM;
    const bool mine = !glu1 || ((wn >= NWN / 2) == (p == 1));
    // the pass's vector rows go out with its first batch's factor blocks
    if (n_runs > 0) dma_vec(p ? ep.vec2 : ep.vec);
#pragma unroll 1
    for (int k0 = 0; k0 < n_runs;) {
      // the batch: runs k0 .. k1 - 1, as many as the factor area holds
      int k1 = k0, used = 0;
      while (k1 < n_runs) {
        const int ch = xm_chunks(rk[k1], cols, ep.use_b_off);
        if (k1 > k0 && used + ch > XM_CHUNKS) break;
        used += ch;
        ++k1;
      }
      // factor blocks: chunk q of the batch at XM + q
      const int nins = (used + 63) / 64;
      for (int t = wave; t < nins; t += NWAVES) {
        const int q = t * 64 + lane;
        int k = k0, base = 0, ch = xm_chunks(rk[k0], cols, ep.use_b_off);
        while (k + 1 < k1 && q >= base + ch) {
          base += ch;
          ++k;
          ch = xm_chunks(rk[k], cols, ep.use_b_off);
        }
        int c = q - base;
        if (c >= ch) c = 0;   // past the batch: any chunk of its last run (unused)
        const int r = rk[k];
        const uint16_t* src;
        if (ep.use_b_off) {
          const int P = max(r >> 3, 1);
          const int n = min(n0 + c / P, N - 1);   // columns past N feed no stored output
          src = lmat + mo[k] + (int64_t)n * r + (c % P) * 8;
        } else {
          const int P = cols / 8 + 1;
          const int rho = c / P;
          int cc = c % P;
          if (cc == P - 1) cc = 0;   // pad chunk
          const int col = min(n0 + cc * 8, N - 8);
          src = lmat + mo[k] + (int64_t)rho * ep.lmat_ld + col;
        }
        dma16v(src, lds_addr(XM + t * 64));
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();

      if (mine) {
        int base = 0;
#pragma unroll 1
        for (int k = k0; k < k1; ++k) {
          const int r = rk[k];
          bool th[4], any = false;   // wave-uniform: 32-row tiles holding rows of run k
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            th[i] = __any(rid[i] == k);
            any |= th[i];
          }
          if (any) {
#pragma unroll 1
            for (int sl = 0; sl * 16 < r; ++sl) {
              const int c = sl * 16 + 8 * half;
              const bool cok = c < r;
              uint4 h[4], l[4], v[NJ];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int row = wm * 128 + i * 32 + m_l;
                const int pc = row * 8 + ((c >> 3) ^ (row & 7));
                h[i] = l[i] = make_uint4(0, 0, 0, 0);
                if (rid[i] == k && cok) {
                  h[i] = XV[pc];
                  l[i] = XL[pc];
                }
              }
              if (ep.use_b_off) {
                const int P = r >> 3;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                  const int col = wn_eff * WN + j * 32 + m_l;
                  v[j] = cok ? XM[base + col * P + (c >> 3)] : make_uint4(0, 0, 0, 0);
                }
              } else {
                // lane: column j*32 + m_l, ranks c .. c + 7 (rows of the staged A_a)
                const int PB = cols + 8;   // bf16 per staged row
                const int q = (lane >> 2) & 3, jj = lane & 3;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                  const int col = wn_eff * WN + j * 32 + 16 * ((lane >> 4) & 1) + 4 * jj;
                  const uint32_t off =
                      (uint32_t)(XM_OFF + base * 16 + ((sl * 16 + 8 * half + q) * PB + col) * 2);
                  const uint2 lo4 = tr_read((const uint4*)X, off);
                  const uint2 hi4 = tr_read((const uint4*)X, off + 4 * PB * 2);
                  v[j] = cok ? make_uint4(lo4.x, lo4.y, hi4.x, hi4.y) : make_uint4(0, 0, 0, 0);
                }
              }
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                if (!th[i]) continue;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                  acc[i][j] = mfma32(as_bf16x8(v[j]), as_bf16x8(h[i]), acc[i][j]);
                  acc[i][j] = mfma32(as_bf16x8(v[j]), as_bf16x8(l[i]), acc[i][j]);
                }
              }
            }
          }
          base += xm_chunks(r, cols, ep.use_b_off);
        }
      }
      __syncthreads();   // every wave is done with the batch (and the pass's vectors)
      k0 = k1;
    }
  }
}

// One 256 x 256 output tile t of gemm_nt_kernel (live_m: live row tiles).
template <int EPI>
__device__ __forceinline__ void gemm_nt_tile(const uint16_t* __restrict__ A,
                                             const uint16_t* __restrict__ B, int M, int N, int K,
                                             int64_t lda, int64_t ldb, const GemmEpi& ep,
                                             int tiles_n, int group_m, int live_m, int t) {
  int tm, tn, g = 0;
  if (ep.g_tile) {
    // grouped: tiles run group by group (group g owns tiles g_tile[g] * tiles_n
    // .. g_tile[g + 1] * tiles_n), row tiles fastest; a group of more than
    // 2 group_m row tiles runs in blocks of group_m row tiles.  The tiles one
    // XCD runs at a time then share their group's weight panels and row
    // panels in its L2
    g = find_bucket_wave(ep.g_tile, ep.n_groups + 1, t / tiles_n);   // whole waves, uniform t
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

  // Opaque per tile: the lane-derived addresses are recomputed for each tile
  // rather than hoisted out of the tile loop and held across the epilogue.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
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

  // Gathered A rows of this wave's DMA (instruction i fills rows 8 (w DMA_PER_OP
  // + i) .. + 7 of a stage; lane L takes row L / 8), loaded first and in one
  // batch: the first DMA waits on them, and nothing else.
  int arow[DMA_PER_OP];
#pragma unroll
  for (int i = 0; i < DMA_PER_OP; ++i)
    arow[i] = min(m0 + (wave * DMA_PER_OP + i) * 8 + (lane >> 3), Mlim - 1);
  if (ep.a_rows) {
#pragma unroll
    for (int i = 0; i < DMA_PER_OP; ++i) arow[i] = ep.a_rows[arow[i]];
  }

  // epilogue row metadata (loaded with the prologue's first stage)
  const int m_l = lane & 31;
  const int n_q = 4 * (lane >> 5);
  int tok[4], ad[4];
  float rs[4];
  int gy[4];          // EPI_LSE / EPI_GRAD: target; EPI_GRAD: dlogp, lse of the rows
  float gd[4], gl[4];
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
    const int rb = min(n0 + (glu1 ? (row & (GBN / 2 - 1)) : row), N - 1);
    const int64_t oa = ep.a_rows ? (int64_t)arow[i] * lda : (int64_t)(arow[i] - m0) * lda;
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
  // The row metadata, issued between the two stages' DMA: it lands with stage
  // 0 (the prologue's wait covers it) and does not delay stage 0.
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
  if (KT > 1) {
#pragma unroll
    for (int i = 0; i < DMA_PER_OP; ++i) dmaA(1, i, baseA + SBK);
#pragma unroll
    for (int i = 0; i < DMA_PER_OP; ++i) dmaB(1, i, bsrc(SBK));
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }

  // LoRA expand tables, built after the first k step, whose barrier has waited
  // for every load so far: built before it, the wait for the row metadata
  // would also wait for the second stage's DMA (issued later), and the first
  // step's MFMAs could not run while that stage lands.  Every wave of the
  // block calls it at that point.
  int x_runs = 0;
  XDesc x_dk{0, 0};
  auto prep = [&]() {
    if (EPI == EPI_BF16 && ep.vec) {
      int vrow[4];   // vector row of each fragment row: its C row, or its position
#pragma unroll
      for (int i = 0; i < 4; ++i) vrow[i] = ep.vec_by_pos ? m0 + wm * 128 + i * 32 + m_l : tok[i];
      x_runs = expand_prep(ep, (char*)g_stage, wave, lane, glu1, ad, vrow, x_dk);
    }
  };

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
  // most of the step to land.  The step's one barrier sits after the third
  // group of its last phase (XBAR), whose remaining groups read the next
  // stage's first slice under their MFMAs (measured against groups 0..6: the
  // q/o GEMM is fastest here, with the DMA phase's issue priority below).
  // sched_barrier keeps the groups in this order.  After the wait and the
  // barrier the next stage is visible and its first slice is read.
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
    constexpr int XBAR = 2;     // group of the last phase that holds the barrier
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cur = q & 1, nxt = cur ^ 1;
      static_assert(G == 2 * DMA_PER_OP, "one DMA per group of the first phase");
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int i = g / NJ, j = g % NJ;
        if (q == 3 && g == XBAR) {
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
        } else if (g >= XBAR) {
          // 4 + NJ reads over the groups after the barrier
#pragma unroll
          for (int t = 0; t < 4 + NJ; ++t) {
            if (t * (G - XBAR) / (4 + NJ) != g - XBAR) continue;
            if (t < 4) fa[nxt][t] = as_bf16x8(An[a_row[t] + cq[0]]);
            else fb[nxt][t - 4] = as_bf16x8(Bn[b_row[t - 4] + cq[0]]);
          }
        }
        // The first phase issues the next stage's DMA: this wave takes issue
        // priority over the other wave of its SIMD for that phase, so the DMA
        // leaves as early as possible and has the most time to land.
        if (q == 0 && g == 0) __builtin_amdgcn_s_setprio(2);
        if (q == 1 && g == 0) __builtin_amdgcn_s_setprio(0);
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
    step(std::integral_constant<int, 0>{}, 0);
    prep();
    for (kt = 1; kt + 2 <= KT; kt += 2) {
      step(std::integral_constant<int, 1>{}, kt);
      step(std::integral_constant<int, 0>{}, kt + 1);
    }
    if (kt < KT) step(std::integral_constant<int, 1>{}, kt);
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
      if (kt == 0) prep();
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
    if (ep.vec) x_tables(ep, glu1, T, x_runs, x_dk);
    __syncthreads();   // every wave is done reading the ring; the run tables are visible
    if (ep.vec) lora_expand(ep, T, n0, N, wave, lane, glu1, x_runs, acc);
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

// Kernel arguments of gemm_nt_kernel, one struct so that the kernel can read
// them back from the argument segment.
struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  int M, N, K;
  int64_t lda, ldb;
  GemmEpi ep;
  int tiles_m, tiles_n, group_m;
};

// Persistent over the tiles: tile ids are XCD-contiguous (XCD x runs a
// contiguous range of them, grouped along M as gemm_nt_tile maps them), and
// the blocks of one XCD take its range round robin.  Grouped launches are
// sized for a bound on the row tiles; the live count comes from the device
// prefix and the live tiles are split evenly over the XCDs, so no XCD is left
// with only dead tiles.  A block's loop ends when its XCD's range is done
// (surplus blocks exit at once).  Each tile reads the arguments afresh from
// the argument segment (scalar loads through a pointer the compiler cannot
// prove loop-invariant): held across the loop they would not fit in the
// scalar registers beside the k loop's own.
template <int EPI>
__global__ __launch_bounds__(GTHREADS, 1) void gemm_nt_kernel(GemmArgs args) {
  typedef const __attribute__((address_space(4))) GemmArgs* KPtr;
  const KPtr kbase = (KPtr)__builtin_amdgcn_kernarg_segment_ptr();
  const int live_m = args.ep.g_tile ? args.ep.g_tile[args.ep.n_groups] : args.tiles_m;
  const int num = live_m * args.tiles_n;
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int per = num >> 3, rem = num & 7;
  const int cnt = per + (xcd < rem ? 1 : 0);
  const int first = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  const int nb = (int)(gridDim.x >> 3) + (xcd < (int)(gridDim.x & 7) ? 1 : 0);   // this XCD's blocks
  for (int j = loc; j < cnt; j += nb) {
    KPtr kp = kbase;
    asm volatile("" : "+s"(kp));
    const GemmArgs& a = *(const GemmArgs*)kp;
    gemm_nt_tile<EPI>(a.A, a.B, a.M, a.N, a.K, a.lda, a.ldb, a.ep, a.tiles_n, a.group_m, live_m,
                      first + j);
    __syncthreads();   // the epilogue's LDS reads are done before the next tile's DMA
  }
}

// ---- few-row GEMM (decode-shaped batches)
//
// With M of a few hundred rows the 256x256 tiles leave most CUs idle (256 rows
// and 4096 columns make 16 blocks) and the product is bound by reading the
// weight once.  Here a block of 4 waves owns a 64 x 64 output tile over the
// whole K -- 256 rows x 4096 columns make 256 blocks, one per CU -- and streams
// its 64 operand rows of each side through a ring of FR_NST LDS-DMA stages of
// k = 128 (32 KB each; steps of 8 MFMAs per wave amortise the per-step wait,
// barrier and DMA issue), so every CU keeps ~96 KB of loads in flight.
// The 4 row tiles of one weight panel run on the same XCD (row tile fastest
// within an XCD's contiguous range), so the panel comes from HBM once and the
// other three read it from that XCD's L2; x is L2-resident.  Per (row tile,
// column tile) pair that is (64 + 64) x K x 2 bytes per CU, the least for 256
// blocks of this shape.
// Each output element is accumulated exactly as in gemm_nt_kernel: one
// v_mfma_f32_32x32x16_bf16 accumulator per 32 x 32 sub-tile with the same
// operand order and lane layout, k in 16-wide slices in increasing order, then
// the LoRA expand per adapter and 16-rank slice (hi, then lo), so a row gets
// the same bits from either kernel (rows of other adapters only receive exact
// zeros).  Plain epilogue only: bf16 store, rows through a_rows / c_rows,
// expand from B_a (use_b_off = 1).
constexpr int FR_TM = 64, FR_TN = 64;      // block tile
constexpr int FR_KH = 2;                   // 64-wide k halves per stage (k = 128 per stage)
constexpr int FR_NST = 5;                  // ring stages (5 x 32 KB)
constexpr int FR_SUB = (FR_TM + FR_TN) * S_CH;     // uint4 per k half of a stage (16 KB)
constexpr int FR_STAGE = FR_KH * FR_SUB;           // uint4 per stage (32 KB)
constexpr int FR_DMA = 4 * FR_KH;          // DMA instructions per wave per stage
__shared__ uint4 fr_ring[FR_NST * FR_STAGE];

// s_waitcnt vmcnt(FR_DMA n): at most n stages of this wave's DMA outstanding
__device__ __forceinline__ void fr_wait(int n) {
  if (n >= 3) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
  else if (n == 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
static_assert(FR_DMA == 8 && FR_NST - 2 <= 3, "fr_wait counts 8 DMA per stage, up to 3 stages");

__global__ __launch_bounds__(256, 1) void gemm_fewrow_kernel(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ B, int M,
                                                             int N, int K, int64_t lda,
                                                             int64_t ldb, GemmEpi ep) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;   // 32-row, 32-column sub-tile of this wave
  const int tiles_m = (M + FR_TM - 1) / FR_TM, tiles_n = (N + FR_TN - 1) / FR_TN;
  const int num = tiles_m * tiles_n;
  const int b = blockIdx.x, xcd = b & 7, loc = b >> 3;
  const int per = num >> 3, rem = num & 7;
  if (loc >= per + (xcd < rem ? 1 : 0)) return;
  const int t = (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
  const int m0 = (t % tiles_m) * FR_TM, n0 = (t / tiles_m) * FR_TN;

  // DMA sources: instruction i = 4 h + j of wave w fills k half h of a stage:
  // rows 8 (2 w + j) .. + 7 of A (j < 2) or of B (j >= 2, j - 2 for the row);
  // lane L lands in row L / 8, physical chunk L % 8, i.e. logical chunk
  // (L % 8) ^ lds_sw(row).  Rows past the edge are clamped: they only feed
  // outputs that are never stored.
  uint32_t off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 8 * (2 * wave + (j & 1)) + (lane >> 3);
    const int chunk = (lane & 7) ^ lds_sw(row);
    if (j < 2) {
      const int ra = min(m0 + row, M - 1);
      const int64_t oa = ep.a_rows ? (int64_t)ep.a_rows[ra] * lda : (int64_t)(ra - m0) * lda;
      off[j] = (uint32_t)((oa + chunk * 8) * 2);
    } else {
      const int rb = min(n0 + row, N - 1);
      off[j] = (uint32_t)(((int64_t)(rb - n0) * ldb + chunk * 8) * 2);
    }
  }
  const uint16_t* baseA = ep.a_rows ? A : A + (int64_t)m0 * lda;
  const uint16_t* baseB = B + (int64_t)n0 * ldb;
  // LDS destination of instruction j within a k half: A rows at offset 0, B
  // rows after the FR_TM A rows
  uint32_t ldsd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    ldsd[j] = __builtin_amdgcn_readfirstlane(
        lds_addr(fr_ring + ((j < 2 ? 0 : FR_TM) + 8 * (2 * wave + (j & 1))) * S_CH));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // only DMA is counted from here on
  const int KT = K / (SBK * FR_KH);   // K is a multiple of 128 here
  auto issue = [&](int s) {
    const uint32_t so = (uint32_t)((s % FR_NST) * FR_STAGE) * 16u;
#pragma unroll
    for (int h = 0; h < FR_KH; ++h) {
      const int k0 = (s * FR_KH + h) * SBK;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dma16s(off[j], (j < 2 ? baseA : baseB) + k0, ldsd[j] + so + (uint32_t)(h * FR_SUB) * 16u);
    }
  };
  // The ring holds FR_NST stages; stage s goes to slot s % FR_NST.  Step kt
  // runs the MFMAs of stage kt on fragments read during step kt - 1, after
  // waiting for stage kt + 1, a barrier and the reads of stage kt + 1, so the
  // LDS latency and the barrier overlap the MFMA chain.  After that barrier
  // every wave has issued the MFMAs of step kt - 1 (so its reads of stage
  // kt - 1 are complete): that slot takes stage kt + FR_NST - 1.
#pragma unroll
  for (int s = 0; s < FR_NST - 1; ++s)
    if (s < KT) issue(s);

  const int frag_row = lane & 31, frag_half = lane >> 5;
  const int ra_l = (wm * 32 + frag_row) * S_CH;             // A row of this lane's fragments
  const int rb_l = (FR_TM + wn * 32 + frag_row) * S_CH;     // B row
  const int sw = lds_sw(frag_row);                          // rows 32 apart share the swizzle
  // two fragment sets: a step's MFMAs read one while the next stage's
  // fragments land in the other (no register copies between steps)
  bf16x8 fa[2][FR_KH][4], fb[2][FR_KH][4];
  auto read_frags = [&](auto S_, int s) {
    constexpr int S = decltype(S_)::value;
#pragma unroll
    for (int h = 0; h < FR_KH; ++h) {
      const uint4* st = fr_ring + (s % FR_NST) * FR_STAGE + h * FR_SUB;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = (2 * q + frag_half) ^ sw;
        fa[S][h][q] = as_bf16x8(st[ra_l + c]);
        fb[S][h][q] = as_bf16x8(st[rb_l + c]);
      }
    }
  };
  f32x16 acc;
#pragma unroll
  for (int g = 0; g < 16; ++g) acc[g] = 0.f;
  fr_wait(min(FR_NST - 2, KT - 1));
  __builtin_amdgcn_s_barrier();   // stage 0 landed for every wave
  read_frags(std::integral_constant<int, 0>{}, 0);
  auto step = [&](auto S_, int kt) {
    constexpr int S = decltype(S_)::value;
    // this step's fragments were read a step ago: wait for them here, where it
    // costs nothing, in a form the compiler sees (s_waitcnt lgkmcnt(0))
    __builtin_amdgcn_s_waitcnt(0xC07F);
    if (kt + 1 < KT) {
      fr_wait(min(FR_NST - 3, KT - 2 - kt));   // stage kt + 1 landed (this wave)
      __builtin_amdgcn_s_barrier();            // ... for every wave; stage kt - 1 consumed by all
      if (kt + FR_NST - 1 < KT) issue(kt + FR_NST - 1);   // into stage kt - 1's slot
      read_frags(std::integral_constant<int, 1 - S>{}, kt + 1);
    }
#pragma unroll
    for (int h = 0; h < FR_KH; ++h)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = mfma32(fb[S][h][q], fa[S][h][q], acc);
  };
  int kt = 0;
  for (; kt + 2 <= KT; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt);
    step(std::integral_constant<int, 1>{}, kt + 1);
  }
  if (kt < KT) step(std::integral_constant<int, 0>{}, kt);

  const int rl = frag_row, half = frag_half;
  const int m = m0 + wm * 32 + rl;
  const int nb = n0 + wn * 32;        // first column of this wave
  const int crow = m < M ? (ep.c_rows ? ep.c_rows[m] : m) : -1;
  if (ep.vec) {
    const int ad = m < M ? ep.adpos[m] : -1;
    const int vrow = ep.vec_by_pos ? m : crow;
    // this row's scaled vector (both planes, every 16-rank slice), loaded once
    constexpr int SL = 4;   // slices of the largest rank (64)
    uint4 hb[SL], lb[SL];
#pragma unroll
    for (int sl = 0; sl < SL; ++sl) {
      const int c = sl * 16 + 8 * half;
      hb[sl] = lb[sl] = make_uint4(0, 0, 0, 0);
      if (ad >= 0 && c < ep.vec_ld) {
        const uint16_t* vp = ep.vec + (int64_t)vrow * ep.vec_ld + c;
        hb[sl] = *(const uint4*)vp;
        lb[sl] = *(const uint4*)(vp + ep.vec_plane);
      }
    }
    // the adapters present in the wave's rows, in increasing order (a
    // wave-uniform walk), XB at a time: their descriptors, then all of their
    // factor slices, are loaded together, so a batch costs two memory round
    // trips rather than two per adapter.  A row changes only in its own
    // adapter's MFMAs (the others add exact zeros), slice by slice, hi then lo.
    auto next_after = [&](int prev) {
      int nxt = ad > prev ? ad : INT32_MAX;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) nxt = min(nxt, __shfl_xor(nxt, o));
      return __builtin_amdgcn_readfirstlane(nxt);
    };
    constexpr int XB = 8;
    int prev = -1;
    for (;;) {
      int as[XB];
      int na = 0;
#pragma unroll
      for (int i = 0; i < XB; ++i) {
        as[i] = next_after(prev);
        if (as[i] != INT32_MAX) {
          prev = as[i];
          na = i + 1;
        } else {
          prev = INT32_MAX - 1;   // later slots find nothing
        }
      }
      if (na == 0) break;
      int64_t boff[XB];
      int rk[XB];
#pragma unroll
      for (int i = 0; i < XB; ++i) {
        boff[i] = 0;
        rk[i] = 0;
        if (i < na) {
          boff[i] = ep.desc[as[i]].b_off;
          rk[i] = ep.desc[as[i]].rank;
        }
      }
      uint4 v[XB][SL];
#pragma unroll
      for (int i = 0; i < XB; ++i) {
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) {
          const int c = sl * 16 + 8 * half;
          const int n = nb + rl;
          v[i][sl] = make_uint4(0, 0, 0, 0);
          if (i < na && c < rk[i] && n < N)
            v[i][sl] = *(const uint4*)(ep.lmat + boff[i] + (int64_t)n * rk[i] + c);
        }
      }
#pragma unroll
      for (int i = 0; i < XB; ++i) {
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) {
          if (i < na && sl * 16 < rk[i]) {
            const bool mine = ad == as[i] && sl * 16 + 8 * half < rk[i];
            const uint4 h = mine ? hb[sl] : make_uint4(0, 0, 0, 0);
            const uint4 lo = mine ? lb[sl] : make_uint4(0, 0, 0, 0);
            acc = mfma32(as_bf16x8(v[i][sl]), as_bf16x8(h), acc);
            acc = mfma32(as_bf16x8(v[i][sl]), as_bf16x8(lo), acc);
          }
        }
      }
      if (na < XB) break;
    }
  }
  if (crow < 0) return;
  // register g of acc: column nb + 8 (g / 4) + 4 half + g % 4
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n = nb + 8 * q + 4 * half;
    if (n < N)
      *(uint2*)(ep.C + (int64_t)crow * ep.ldc + n) =
          make_uint2(pack2bf(acc[4 * q], acc[4 * q + 1]), pack2bf(acc[4 * q + 2], acc[4 * q + 3]));
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
  if (EPI == EPI_BF16 && ep.vec &&
      (ep.vec_ld < 8 || ep.vec_ld > 64 || ep.vec_ld % 8 || ep.vec_plane % 8 || N % 8 ||
       !ep.desc || !ep.lmat || !ep.adpos || ((ep.glu == 1 || ep.k_split > 0) && ep.vec2 && (!ep.desc2 || !ep.lmat2)))) {
    set_error("gemm: LoRA expand needs vec_ld in 8..64 (a multiple of 8), 16-byte aligned "
              "planes, N a multiple of 8 and both factor sets");
    return LORA_E_INVALID_ARG;
  }
  if (ep.k_split > 0 && (ep.k_split % SBK || ep.k_split >= K || !ep.B2)) {
    set_error("gemm: K split %d must be a multiple of %d below K = %d, with B2", ep.k_split, SBK, K);
    return LORA_E_INVALID_ARG;
  }
  if (tiles_m <= 0) return LORA_OK;
  if ((int64_t)tiles_m * tiles_n > INT32_MAX) {   // tile ids are 32-bit in the kernels
    set_error("gemm: %lld x %lld output tiles exceed 2^31", (long long)tiles_m, (long long)tiles_n);
    return LORA_E_UNSUPPORTED;
  }
  // few rows (a plain product, or with the expand from B_a): the few-row kernel
  // keeps every CU busy where the 256x256 tiles would not
  if constexpr (EPI == EPI_BF16) {
    if (!ep.g_tile && ep.glu == 0 && ep.k_split == 0 && !ep.rowscale &&
        (!ep.vec || ep.use_b_off) && (int64_t)tiles_m * tiles_n < 64 && K % 128 == 0 &&
        N % 4 == 0 && ep.ldc % 4 == 0) {
      hipLaunchKernelGGL(gemm_fewrow_kernel, dim3((unsigned)(cdiv(M, FR_TM) * cdiv(N, FR_TN))),
                         dim3(256), 0, s, A, B, M, N, K, lda, ldb, ep);
      return launch_check("gemm_fewrow");
    }
  }
  if (group_m <= 0) group_m = pick_group_m(tiles_m);
  if (group_m > tiles_m) group_m = tiles_m;
  // operand tiles are static LDS objects: no dynamic LDS
  // one resident block per CU (the LDS block is a whole CU's), each looping over tiles
  const int grid = (int)std::min<int64_t>((int64_t)tiles_m * tiles_n, std::max(device_cus(), 8));
  const GemmArgs args{A, B, M, N, K, lda, ldb, ep, tiles_m, tiles_n, group_m};
  hipLaunchKernelGGL(gemm_nt_kernel<EPI>, dim3(grid), dim3(GTHREADS), 0, s, args);
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
