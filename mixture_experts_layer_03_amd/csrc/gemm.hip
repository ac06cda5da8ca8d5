// Grouped expert GEMMs on gfx950 MFMA (bf16 in, fp32 accumulate) with fused
// epilogues, and the fp32 forward fallback.
//
// The pages: experts run as one grouped matmul over the tokens sorted by
// expert ("Halo's 2.8x over TRL is not a kernel, and its own benchmark proves
// it", section "Where the gap actually is"), with a fused SwiGLU ("grouped
// GEMM and fused SwiGLU", "Halo: Frontier-Lab Training for Everyone", section
// "Novel model integration example"), over fused 3-D expert weights (section
// "One trainer architecture, one parallelism stack").  A fused SwiGLU kernel
// overflowed once a router put 745k tokens on one GPU's experts (section
// "Some of the hard problems along the way"); every element offset here is
// 64-bit.
//
// One kernel template serves six GEMMs.  Each computes, per expert, an output
// tile D[p][q] = sum_k P[p][k] * Q[q][k]:
//   kind        P (MFMA rows, output-contiguous)   Q (MFMA cols)        K
//   FWD_GU      W_gu[e] gate|up rows (paired)       X_perm rows of e     d
//   FWD_DOWN    W_down[e] rows                      H rows of e          f
//   BWD_DH      W_down[e] columns (transposed)      dY_perm rows of e    d
//   BWD_DX      W_gu[e] columns (transposed)        dGU rows of e        2f
//   BWD_DWDOWN  H columns (transposed, rows of e)   w*dY_perm columns    M_e
//   BWD_DWGU    X_perm columns (transposed)         dGU columns          M_e
// "transposed" operands are stored with the GEMM's K as their slow index; the
// loader reads 8x8 bf16 blocks with 16-byte loads along the fast index and
// transposes them in registers, so LDS always holds K-contiguous rows.
//
// MFMA: v_mfma_f32_16x16x32_bf16.  Lane l supplies row l%16 of a 16-row
// fragment with the 8 bf16 of 16-byte chunk (l/16) of the 32-wide k step (the
// same chunk map for both operands, so the dot products pair correctly); the
// result holds D[4*(l/16)+v][l%16], v = 0..3.
#include <mutex>

#include "moe_internal.h"

namespace moe {

enum GemmKind { FWD_GU = 0, FWD_DOWN = 1, BWD_DH = 2, BWD_DX = 3, BWD_DWDOWN = 4, BWD_DWGU = 5 };


struct GemmArgs {
  // operands
  const bf16_t *x_perm, *w_gu, *w_down, *h, *gu, *dy_perm, *dgu, *s_perm;
  const float *row_scale;      // [R] or null
  const int32_t *offsets;      // [E+1]
  const int32_t *tile_start;   // [E+1] (token-tiled kinds)
  int32_t *counters;           // [8] per-XCD tile counters, zero at launch (token-tiled kinds)
  // outputs
  bf16_t *o_gu, *o_h, *o_y, *o_dgu, *o_dx;
  float *o_dw, *o_drs;         // dw: [E, Qdim, Pdim]; drs partials [R, PT*WP]
  // grouped LoRA (token GEMMs with one extra K stage of width lora_r):
  //   FWD_GU   P: B_gu [E,2f,r] rows   Q: z_gu [R,r] rows
  //   FWD_DOWN P: B_dn [E,d,r] rows    Q: z_dn [R,r] rows
  //   BWD_DH   P: A_dn [E,r,f] (transposed, like W_down)   Q: u_dn [R,r] rows
  //   BWD_DX   P: A_gu [E,r,d] (transposed, like W_gu)     Q: u_gu [R,r] rows
  const bf16_t *lora_p, *lora_q;
  int lora_r;
  // gathered operands (GATHER kernels): token rows of an unpermuted
  // [gx_rows, ld] source, row r of the expert-sorted order being token
  // row_to_slot[r] / k (kmagic = floor(2^32 / k) + 1):
  //   FWD_GU   Q: X rows        BWD_DH   Q: dY rows
  //   BWD_DWGU P: X columns (its k-rows are tokens)
  const bf16_t *gx;
  const int32_t *row_to_slot;
  uint64_t kmagic;
  int64_t gx_rows;
  int E, d, f;
  const int32_t *wg_bounds;    // weight-gradient kinds: [9] per-XCD chunk bounds, or null
  int PT;                      // tiles along P
  int QT;                      // tiles along Q (weight-gradient kinds)
  int nlogical;                // weight-gradient kinds: E*PT*QT
};

// ------------------------------------------------------------------ helpers

#define LDS_AS __attribute__((address_space(3)))
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Raw buffer resource (gfx9 V#) over [base, base + bytes): loads at offsets
// >= bytes return zeros, so tile edges and K tails need no branches.
__device__ __forceinline__ u32x4_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4_t r;
  r[0] = (uint32_t)a;
  r[1] = (uint32_t)(a >> 32) & 0xffffu;   // stride 0
  r[2] = bytes;                           // num_records
  r[3] = 0x00020000u;                     // raw dword access
  return r;
}
constexpr uint32_t kOOB = 0x80000000u;   // an offset past any resource: reads zero

// One 16-byte chunk per lane from global memory straight into LDS; the wave's
// 64 chunks land contiguously at dst (lane l at dst + 16*l).  Written as
// inline assembly so that the compiler does not guard later LDS reads of
// other buffers with waits for these loads; the kernel waits for them itself
// (wait_vm_lgkm0) before the barrier that publishes a stage.
__device__ __forceinline__ void dma16_at(u32x4_t rs, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rs)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)((const LDS_AS void *)p);
}
__device__ __forceinline__ void dma16(u32x4_t rs, u32x4_t *dst, uint32_t voff) {
  dma16_at(rs, lds_addr(dst), voff);
}
// The same with 4 bytes per lane (lane l at dst + 4*l).
__device__ __forceinline__ void dma4_at(u32x4_t rs, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rs)
               : "memory", "m0");
}

// Token of top-k slot `slot` (slot / k): exact for slot * k < 2^32 with
// kmagic = floor(2^32 / k) + 1 (the rounding error slot / 2^32 stays below
// the 1/k gap to the next multiple).
__device__ __forceinline__ uint32_t slot_token(int slot, uint64_t kmagic) {
  return (uint32_t)(((uint64_t)(uint32_t)slot * kmagic) >> 32);
}

// s_waitcnt with vmcnt <= n (n < 64) and lgkmcnt = 0 (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// ---------------------------------------------------------------- LDS layouts
//
// K-contiguous operand tile: ROWS rows x BK k (BK/8 chunks of 16 bytes per
// row).  Chunk ch of row r sits at slot r*CPR + (ch ^ kc_swz(r)), with the
// swizzle taken from row bits 1.. : measured on gfx950, 16-byte reads of 16
// consecutive rows (one chunk each) then run at the conflict-free rate, which
// a swizzle on bits 2.. (one 256-byte line per XOR value) does not reach.
// The swizzle repeats every 16 rows.
template <int BK>
__device__ __forceinline__ int kc_swz(int row) { return (row >> 1) % (BK / 8); }

template <int BK>
__device__ __forceinline__ int kc_slot(int row, int ch) {
  return row * (BK / 8) + (ch ^ kc_swz<BK>(row));
}

// Transposed operand tile: BK k-rows x COLS columns (COLS*2 bytes per k-row).
// The 32-byte column block cb of k-row r sits at cb ^ tr_swz(r): the 16 k-rows
// that one transpose read of a wave touches (8g + 0..3 for g = 0..3, or +4)
// land on 8 distinct 32-byte bank groups per half-wave.
__device__ __forceinline__ int tr_swz(int r) { return (r & 3) | (((r >> 3) & 1) << 2); }

// Issue the direct-to-LDS loads of one BK-wide K stage of a ROWS-row operand
// tile; every wave issues ROWS*BK/(512*NW) instructions of 1 KB.  All
// arguments but lane are wave-uniform.
//   K-contiguous: element (row i, k) at base[i*ld + k] (rows >= ROWS/2 of a
//     paired tile from base2); rows_valid rows and kvalid k exist.
//   transposed:   element (row i, k) at base[k*ld + i]; rows_valid columns
//     and kvalid k-rows exist.
template <int ROWS, bool TRANS, bool PAIRED, int NW, int BK>
__device__ __forceinline__ void issue_stage(const bf16_t *base, const bf16_t *base2, int ld,
                                            int rows_valid, int kvalid, int k0, u32x4_t *tile,
                                            int wave, int lane) {
  constexpr int NI = ROWS * BK / 512 / NW;
  static_assert(NI >= 1 && NI * 512 * NW == ROWS * BK, "tile splits evenly over the waves");
  if (!TRANS) {
    constexpr int CPR = BK / 8;             // chunks per row
    constexpr int RPI = 64 / CPR;           // rows per instruction
    constexpr int half_rows = PAIRED ? ROWS / 2 : ROWS;
    // a wave's NI instructions cover RPI*NI consecutive rows, all in one half
    static_assert(!PAIRED || (ROWS / 2 / RPI) % NI == 0, "paired halves align with waves");
    const bool second = PAIRED && wave * NI >= ROWS / 2 / RPI;
    const int rv = min(rows_valid, half_rows);
    const uint32_t bytes = rv > 0 ? (uint32_t)rv * (uint32_t)ld * 2u : 0u;
    const u32x4_t rs = make_rsrc(second ? base2 : base, bytes);
    const int row_shift = second ? ROWS / 2 : 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = wave * NI + i;          // rows RPI*q .. RPI*q + RPI-1
      const int row = RPI * q + lane / CPR;
      const int ch = (lane % CPR) ^ kc_swz<BK>(row);
      const int k = k0 + ch * 8;
      const uint32_t off =
          k < kvalid ? ((uint32_t)(row - row_shift) * (uint32_t)ld + (uint32_t)k) * 2u : kOOB;
      dma16(rs, tile + q * 64, off);
    }
  } else {
    constexpr int C16 = ROWS / 8;           // 16-byte chunks per k-row
    // The resource ends right after the tile's last valid element (column
    // cols-1 of k-row krows-1): columns past the valid ones read the next
    // k-row's data (finite values feeding only masked outputs) or zeros past
    // the end, never memory beyond the tensor.
    const int krows = min(BK, kvalid - k0);
    const int cols = min(rows_valid, ROWS);
    const uint32_t bytes = (krows > 0 && cols > 0)
                               ? ((uint32_t)(krows - 1) * (uint32_t)ld + (uint32_t)cols) * 2u
                               : 0u;
    const u32x4_t r1 = make_rsrc(base + (int64_t)k0 * ld, bytes);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = wave * NI + i;
      const int lin = q * 64 + lane;        // 16-byte slot inside the tile
      const int kr = lin / C16;
      const int pc = lin % C16;
      const int c16 = pc ^ (tr_swz(kr) << 1);
      const uint32_t off = ((uint32_t)kr * (uint32_t)ld + (uint32_t)c16 * 8u) * 2u;
      dma16(r1, tile + q * 64, off);
    }
  }
}

// Loop-invariant byte offsets of one wave's direct-to-LDS loads of an
// operand, for every stage and tile of a kind (the leading dimension ld is
// fixed per kind); the stage's k0 moves the resource base instead.
//   K-contiguous: row part + swizzled 16-byte chunk of the stage's k range.
//   transposed:   k-row part + swizzled 16-byte column chunk.
// Instruction i + 2 covers the rows (k-rows) 2*RPI (2*64/C16) further on,
// where both swizzles repeat, so its offset is instruction i's plus `stride`:
// only the first two offsets are kept.
template <int ROWS, bool TRANS, bool PAIRED, int NW, int BK>
__device__ __forceinline__ void init_voff(int ld, int wave, int lane,
                                          uint32_t (&voff)[(ROWS * BK / 512 / NW) < 2
                                                               ? (ROWS * BK / 512 / NW)
                                                               : 2],
                                          uint32_t &stride) {
  constexpr int NI = ROWS * BK / 512 / NW;
  constexpr int NV = NI < 2 ? NI : 2;
  if (!TRANS) {
    constexpr int CPR = BK / 8, RPI = 64 / CPR;
    static_assert((2 * RPI) % (2 * CPR) == 0, "chunk swizzle repeats after two instructions");
    const bool second = PAIRED && wave * NI >= ROWS / 2 / RPI;
    const int row_shift = second ? ROWS / 2 : 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int q = wave * NI + i;
      const int row = RPI * q + lane / CPR;
      const int ch = (lane % CPR) ^ kc_swz<BK>(row);
      voff[i] = ((uint32_t)(row - row_shift) * (uint32_t)ld + (uint32_t)ch * 8u) * 2u;
    }
    stride = (uint32_t)(2 * RPI) * (uint32_t)ld * 2u;
  } else {
    constexpr int C16 = ROWS / 8;
    // k-rows 8w + 2i + lane/32 (i < 4): adding 4 keeps bits 0, 1 and 3
    static_assert((ROWS == 256 && NI <= 4) || (ROWS == 128 && NI <= 2),
                  "column swizzle repeats after two instructions");
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int lin = (wave * NI + i) * 64 + lane;
      const int kr = lin / C16;
      const int c16 = (lin % C16) ^ (tr_swz(kr) << 1);
      voff[i] = ((uint32_t)kr * (uint32_t)ld + (uint32_t)c16 * 8u) * 2u;
    }
    stride = (uint32_t)(128 / C16) * (uint32_t)ld * 2u;
  }
}

// Plan one operand's loads for the stage at k0, with the offsets of
// init_voff: this wave's instruction i then loads with resource rs into LDS
// address m + i*step.  Only the resource (base and byte count, wave-uniform)
// changes per stage.  A K-contiguous stage that ends past kvalid (a K tail)
// is issued here by issue_stage, which masks each lane's chunk; its planned
// loads then read nothing (byte count 0) into the spare LDS slot `dummy`.
template <int ROWS, bool TRANS, bool PAIRED, int NW, int BK>
__device__ __forceinline__ void plan_operand(const bf16_t *base, const bf16_t *base2, int ld,
                                             int rows_valid, int kvalid, int k0, u32x4_t *tile,
                                             int wave, int lane, uint32_t dummy, u32x4_t &rs,
                                             uint32_t &m, uint32_t &step) {
  constexpr int NI = ROWS * BK / 512 / NW;
  m = lds_addr(tile + wave * NI * 64);
  step = 1024;
  if (!TRANS) {
    if (k0 + BK > kvalid) {
      issue_stage<ROWS, TRANS, PAIRED, NW, BK>(base, base2, ld, rows_valid, kvalid, k0, tile, wave,
                                               lane);
      rs = make_rsrc(base, 0);
      m = dummy;
      step = 0;
      return;
    }
    // Rows past rows_valid start at or beyond the byte count and read zeros;
    // valid rows end inside it (k0 + BK <= kvalid = ld).
    constexpr int CPR = BK / 8, RPI = 64 / CPR;
    constexpr int half_rows = PAIRED ? ROWS / 2 : ROWS;
    const bool second = PAIRED && wave * NI >= ROWS / 2 / RPI;
    const int rv = min(rows_valid, half_rows);
    const uint32_t bytes = rv > 0 ? ((uint32_t)rv * (uint32_t)ld - (uint32_t)k0) * 2u : 0u;
    rs = make_rsrc((second ? base2 : base) + k0, bytes);
  } else {
    // k-rows past the K range start at or beyond the byte count (ld >= cols)
    const int krows = min(BK, kvalid - k0);
    const int cols = min(rows_valid, ROWS);
    const uint32_t bytes = (krows > 0 && cols > 0)
                               ? ((uint32_t)(krows - 1) * (uint32_t)ld + (uint32_t)cols) * 2u
                               : 0u;
    rs = make_rsrc(base + (int64_t)k0 * ld, bytes);
  }
}

// Gathered K-contiguous operand: byte offsets (from the stage's k0) of this
// wave's loads of tile rows q0.. of an expert segment, each the row of its
// token in the [rows, ld] source; rows past the segment read nothing.  The
// LDS placement is that of issue_stage.
template <int ROWS, int NW, int BK>
__device__ __forceinline__ void gather_rows_voff(const GemmArgs &a, int seg0, int q0, int Me,
                                                 int ld, int wave, int lane,
                                                 uint32_t (&voff)[ROWS * BK / 512 / NW]) {
  constexpr int NI = ROWS * BK / 512 / NW, CPR = BK / 8, RPI = 64 / CPR;
  int slot[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = q0 + RPI * (wave * NI + i) + lane / CPR;
    slot[i] = q < Me ? a.row_to_slot[(int64_t)seg0 + q] : -1;
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = RPI * (wave * NI + i) + lane / CPR;
    const int ch = (lane % CPR) ^ kc_swz<BK>(row);
    voff[i] = slot[i] >= 0
                  ? (slot_token(slot[i], a.kmagic) * (uint32_t)ld + (uint32_t)ch * 8u) * 2u
                  : kOOB;
  }
}

// Plan a gathered K-contiguous stage at k0 (offsets from gather_rows_voff):
// the resource spans the whole source from column k0.  A stage past kvalid
// (K tail) is issued here with each lane's chunk masked, and its planned
// loads then read nothing into `dummy`.
template <int ROWS, int NW, int BK>
__device__ __forceinline__ void plan_gather_rows(const GemmArgs &a, int ld, int kvalid, int k0,
                                                 u32x4_t *tile, int wave, int lane,
                                                 uint32_t dummy,
                                                 const uint32_t (&voff)[ROWS * BK / 512 / NW],
                                                 u32x4_t &rs, uint32_t &m, uint32_t &step) {
  constexpr int NI = ROWS * BK / 512 / NW, CPR = BK / 8, RPI = 64 / CPR;
  rs = make_rsrc(a.gx + k0, (uint32_t)((a.gx_rows * ld - k0) * 2));
  m = lds_addr(tile + wave * NI * 64);
  step = 1024;
  if (k0 + BK > kvalid) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = RPI * (wave * NI + i) + lane / CPR;
      const int ch = (lane % CPR) ^ kc_swz<BK>(row);
      dma16(rs, tile + (wave * NI + i) * 64, k0 + ch * 8 < kvalid ? voff[i] : kOOB);
    }
    rs = make_rsrc(a.gx, 0);
    m = dummy;
    step = 0;
  }
}

// MFMA operand fragments (v_mfma_f32_16x16x32_bf16 A/B layout): rows
// r0..r0+15 of a tile, lane l gets row r0 + l%16 with the 8 k-values of
// 16-byte chunk l/16 of the 32-wide k step.
//
// K-contiguous tile: byte offset of the lane's chunk for rows r0.. at k step
// ks.  Fragments 16*m rows further sit 16*m*CPR slots further (the chunk
// swizzle repeats every 16 rows).
template <int BK>
__device__ __forceinline__ uint32_t kc_frag_off(int r0, int ks, int lane) {
  return (uint32_t)kc_slot<BK>(r0 + (lane & 15), ks * 4 + (lane >> 4)) * 16u;
}

// Transposed tile: byte offset of the lane's first transpose read for
// columns c0..c0+15 (c0 a multiple of 16) at k step 0.  Lane j of each
// 16-lane group g reads k-row 8g + j/4, columns c0 + 4*(j%4) .. +3; after the
// transpose, lane j holds column c0 + j for those 4 k-rows.  The second read
// is 4 k-rows further (same swizzle), k step ks is 32 k-rows further.
template <int ROWS>
__device__ __forceinline__ uint32_t tr_frag_off(int c0, int lane) {
  const int j = lane & 15, g = lane >> 4;
  const int kr = 8 * g + (j >> 2);
  return (uint32_t)(kr * (ROWS * 2) + (((c0 >> 4) ^ tr_swz(kr)) << 5) + (j & 3) * 8);
}

// Row offset of fragment i from the wave's first fragment (paired tiles put
// the wave's up-projection fragments in the second half).
template <bool PAIRED, int ROWS, int F>
__device__ constexpr int frag_delta(int i) {
  return PAIRED ? (i < F / 2 ? 16 * i : ROWS / 2 + 16 * (i - F / 2)) : 16 * i;
}

// Fragment i at k step ks of the operand region sb of a stage; rd holds the
// lane offsets (per k step if K-contiguous, per fragment if transposed).
template <bool TRANS, bool PAIRED, int ROWS, int BK, int F, int NR>
__device__ __forceinline__ bf16x8_t frag_at(const LDS_AS char *sb, const uint32_t (&rd)[NR], int i,
                                            int ks) {
  if constexpr (TRANS) {
    const LDS_AS char *p = sb + rd[i] + ks * (32 * ROWS * 2);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4_t *)(p));
    const s16x4_t hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4_t *)(p + 4 * (ROWS * 2)));
    typedef short s16x8_t __attribute__((ext_vector_type(8)));
    const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  } else {
    constexpr int CPR = BK / 8;
    static_assert(NR <= 2, "one or two k steps per stage");
    const int delta = frag_delta<PAIRED, ROWS, F>(i);
    const uint32_t r = (NR == 2 && ks) ? rd[NR - 1] : rd[0];
    return as_bf16x8(*(const LDS_AS u32x4_t *)(sb + r + delta * (CPR * 16)));
  }
}

template <int KIND> struct KindTraits;
template <> struct KindTraits<FWD_GU>     { static constexpr bool PT_ = false, QT_ = false, PAIRED = true,  WG = false; };
template <> struct KindTraits<FWD_DOWN>   { static constexpr bool PT_ = false, QT_ = false, PAIRED = false, WG = false; };
template <> struct KindTraits<BWD_DH>     { static constexpr bool PT_ = true,  QT_ = false, PAIRED = false, WG = false; };
template <> struct KindTraits<BWD_DX>     { static constexpr bool PT_ = true,  QT_ = false, PAIRED = false, WG = false; };
template <> struct KindTraits<BWD_DWDOWN> { static constexpr bool PT_ = true,  QT_ = true,  PAIRED = false, WG = true; };
template <> struct KindTraits<BWD_DWGU>   { static constexpr bool PT_ = true,  QT_ = true,  PAIRED = false, WG = true; };

// ------------------------------------------------------------------ tiles
//
// One output tile of a grouped GEMM and the operands that feed it.  All fields
// are wave-uniform.
struct Tile {
  int e, seg0, Me, p_tile, q_tile, p0, q0, nk;
  const bf16_t *pb, *pb2, *qb;
  int pld, prv, pkv, qld, qrv, qkv;
  const bf16_t *lpb, *lpb2, *lqb;   // LoRA stage operands (last stage of the tile)
  int lpld;
};


// Logical tile L -> Tile.  s_off / s_ts: offsets[E+1] and tile_start[E+1]
// staged in LDS.
template <int KIND, int BP, int BQ, int BK, bool LORA = false>
__device__ __forceinline__ Tile make_tile(const GemmArgs &a, const int *s_off, const int *s_ts,
                                          int L) {
  using KT = KindTraits<KIND>;
  Tile t;
  if (KT::WG) {
    // Weight gradients: (expert, Q-tile, P-tile) with the P-tile fastest:
    // the tiles in flight on one XCD share their Q operand slab and walk the
    // expert's P slabs together (measured on the gpt-oss-20b-like workload:
    // the same time as the Q-fastest order with half its fetched bytes; bands
    // of 4 P-tiles per Q sweep were 12% slower).
    const int per_e = a.PT * a.QT;
    t.e = L / per_e;
    const int rem = L - t.e * per_e;
    t.q_tile = rem / a.PT;
    t.p_tile = rem - t.q_tile * a.PT;
    t.seg0 = s_off[t.e];
    t.Me = s_off[t.e + 1] - t.seg0;
  } else {
    // Token GEMMs: (expert, P-tile, Q-tile) with the expert's token tiles
    // fastest, so they share each weight slab in L2.
    int lo = 0, hi = a.E;   // largest e with tile_start[e] <= L
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_ts[mid] <= L) lo = mid; else hi = mid;
    }
    t.e = lo;
    t.seg0 = s_off[t.e];
    t.Me = s_off[t.e + 1] - t.seg0;
    const int qt_e = (t.Me + BQ - 1) / BQ;
    const int rem = L - s_ts[t.e];
    t.p_tile = rem / qt_e;
    t.q_tile = rem - t.p_tile * qt_e;
  }
  t.e = __builtin_amdgcn_readfirstlane(t.e);
  t.p_tile = __builtin_amdgcn_readfirstlane(t.p_tile);
  t.q_tile = __builtin_amdgcn_readfirstlane(t.q_tile);
  t.seg0 = __builtin_amdgcn_readfirstlane(t.seg0);
  t.Me = __builtin_amdgcn_readfirstlane(t.Me);
  const int d = a.d, f = a.f, e = t.e, seg0 = t.seg0, Me = t.Me;
  const int64_t f2 = 2 * (int64_t)f;
  t.p0 = t.p_tile * (KT::PAIRED ? BP / 2 : BP);
  t.q0 = t.q_tile * BQ;
  const int p0 = t.p0, q0 = t.q0;
  t.pb2 = nullptr;
  int K = 0;
  if (KIND == FWD_GU) {
    const bf16_t *W = a.w_gu + (int64_t)e * f2 * d;
    t.pb = W + (int64_t)p0 * d; t.pb2 = W + ((int64_t)f + p0) * d; t.pld = d; t.prv = f - p0; t.pkv = d;
    t.qb = a.x_perm + ((int64_t)seg0 + q0) * d; t.qld = d; t.qrv = Me - q0; t.qkv = d;
    K = d;
  } else if (KIND == FWD_DOWN) {
    const bf16_t *W = a.w_down + (int64_t)e * d * f;
    t.pb = W + (int64_t)p0 * f; t.pld = f; t.prv = d - p0; t.pkv = f;
    t.qb = a.h + ((int64_t)seg0 + q0) * f; t.qld = f; t.qrv = Me - q0; t.qkv = f;
    K = f;
  } else if (KIND == BWD_DH) {
    const bf16_t *W = a.w_down + (int64_t)e * d * f;
    t.pb = W + p0; t.pld = f; t.prv = f - p0; t.pkv = d;
    t.qb = a.dy_perm + ((int64_t)seg0 + q0) * d; t.qld = d; t.qrv = Me - q0; t.qkv = d;
    K = d;
  } else if (KIND == BWD_DX) {
    const bf16_t *W = a.w_gu + (int64_t)e * f2 * d;
    t.pb = W + p0; t.pld = d; t.prv = d - p0; t.pkv = (int)f2;
    t.qb = a.dgu + ((int64_t)seg0 + q0) * f2; t.qld = (int)f2; t.qrv = Me - q0; t.qkv = (int)f2;
    K = (int)f2;
  } else if (KIND == BWD_DWDOWN) {
    t.pb = a.h + (int64_t)seg0 * f + p0; t.pld = f; t.prv = f - p0; t.pkv = Me;
    t.qb = a.s_perm + (int64_t)seg0 * d + q0; t.qld = d; t.qrv = d - q0; t.qkv = Me;
    K = Me;
  } else {   // BWD_DWGU
    t.pb = a.x_perm + (int64_t)seg0 * d + p0; t.pld = d; t.prv = d - p0; t.pkv = Me;
    t.qb = a.dgu + (int64_t)seg0 * f2 + q0; t.qld = (int)f2; t.qrv = (int)(f2 - q0); t.qkv = Me;
    K = Me;
  }
  if (!t.pb2) t.pb2 = t.pb;
  t.nk = (K + BK - 1) / BK;
  if constexpr (LORA) {
    // one more K stage: the rank-r product with the LoRA factors
    const int r = a.lora_r;
    t.lqb = a.lora_q + ((int64_t)seg0 + q0) * r;
    if (KIND == FWD_GU) {
      const bf16_t *B = a.lora_p + (int64_t)e * f2 * r;
      t.lpb = B + (int64_t)p0 * r; t.lpb2 = B + ((int64_t)f + p0) * r; t.lpld = r;
    } else if (KIND == FWD_DOWN) {
      t.lpb = a.lora_p + ((int64_t)e * d + p0) * r; t.lpb2 = t.lpb; t.lpld = r;
    } else if (KIND == BWD_DH) {
      t.lpb = a.lora_p + (int64_t)e * r * f + p0; t.lpb2 = t.lpb; t.lpld = f;
    } else {   // BWD_DX
      t.lpb = a.lora_p + (int64_t)e * r * d + p0; t.lpb2 = t.lpb; t.lpld = d;
    }
    t.nk += 1;
  }
  return t;
}

// ------------------------------------------------------------------ epilogues

// Exchange between the 16-lane rows 2k and 2k+1 of a wave (lanes l and
// l ^ 16), x0 and x1 being a lane's words of two fragments: a lane of an
// even row keeps its x0 and takes its partner's x0, a lane of an odd row
// takes its partner's x1 and keeps its x1.  Per 16-lane row r (x[r] the
// words of row r): out0 = (x0[0], x1[0], x0[2], x1[2]), out1 = (x0[1], x1[1],
// x0[3], x1[3]): gfx950's v_permlane16_swap, one instruction per word pair.
__device__ __forceinline__ void pair_rows(uint32_t x0, uint32_t x1, uint32_t &out0,
                                          uint32_t &out1) {
  const auto sw = __builtin_amdgcn_permlane16_swap(x0, x1, false, false);
  out0 = sw[0];
  out1 = sw[1];
}


// h = silu(g) u from the stored (bf16) g and u, in fp32, before its own bf16
// store.  The forward's SwiGLU epilogue and the backward's dSwiGLU epilogue
// both form it with this one expression, so the backward recomputes the
// stored H bit for bit instead of loading it.
__device__ __forceinline__ float swiglu_h(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

//
// Lane holds D[prow[i] + 4*(lane/16) + v][qrow[j] + lane%16].
// Per-wave LDS slot of the down and dX epilogues (128 x 64 waves): 16 token
// rows x 64 bf16 columns, rows padded to 144 bytes.
constexpr int kEpiPitch = 144, kEpiSlot = 16 * kEpiPitch;
template <int KIND, int FP>
constexpr bool epi_via_lds() { return (KIND == FWD_DOWN || KIND == BWD_DX) && FP == 8; }

template <int KIND, int FP, int FQ, int WP>
__device__ __forceinline__ void epilogue(const GemmArgs &a, const Tile &t, f32x4_t (&acc)[FP][FQ],
                                         const int (&prow)[FP], const int (&qrow)[FQ], int lane,
                                         int wp, LDS_AS char *epi) {
  const int d = a.d, f = a.f;
  const int64_t f2 = 2 * (int64_t)f;
  const int er = 4 * (lane >> 4);
  const int ec = lane & 15;
  const int seg0 = t.seg0, Me = t.Me, p0 = t.p0, q0 = t.q0;
  // Lane (g, c) of a fragment holds 4 consecutive P columns (4g..4g+3) of
  // token row c.  In the tiles of 64 x 64 waves (the gathered gate/up and the
  // dH GEMMs), fragments 16 columns apart trade 16-lane rows (pair_rows):
  // lane group g then holds 8 consecutive columns of its row, from 8*sig(g)
  // in the pair's 32 with sig = (0, 2, 1, 3), and a 16-byte access covers 16
  // rows x 64 B instead of 16 rows x 32 B.  (Measured on MI355X: the 4-column
  // stores cost the gate/up GEMM 11-21% of its time, the down and dX GEMMs
  // 6-33%.  In the 128 x 64 waves of those 256 x 256 tiles the exchange
  // pushes the kernels past 256 registers -- 270-340 bytes of spills -- so
  // they keep the 4-column stores.)
  const int grp = lane >> 4;
  const int sig = ((grp & 1) << 1) | (grp >> 1);
  if (KIND == FWD_GU && FP == 4) {
    // gate units are fragments 0, 1, their up features 2, 3
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      const int q = q0 + qrow[j] + ec;
      const int64_t r = (int64_t)seg0 + q;
#pragma unroll
      for (int i = 0; i < FP / 2; i += 2) {   // one pair
        float g[8], u[8], hv[8];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float g0 = acc[i][j][v], g1 = acc[i + 1][j][v];
          const float u0 = acc[i + FP / 2][j][v], u1 = acc[i + 1 + FP / 2][j][v];
          uint32_t ga, gb, ua, ub;
          pair_rows(__float_as_uint(g0), __float_as_uint(g1), ga, gb);
          pair_rows(__float_as_uint(u0), __float_as_uint(u1), ua, ub);
          g[v] = __uint_as_float(ga);
          g[4 + v] = __uint_as_float(gb);
          u[v] = __uint_as_float(ua);
          u[4 + v] = __uint_as_float(ub);
        }
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          g[v] = round_bf16(g[v]);
          u[v] = round_bf16(u[v]);
          hv[v] = swiglu_h(g[v], u[v]);
        }
        const int n = p0 + prow[i] + 8 * sig;   // gate feature; up feature = f + n
        if (q >= Me || n >= f) continue;
        if (a.o_gu) {
          *reinterpret_cast<u32x4_t *>(a.o_gu + r * f2 + n) =
              u32x4_t{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                      pack_bf16x2(g[6], g[7])};
          *reinterpret_cast<u32x4_t *>(a.o_gu + r * f2 + f + n) =
              u32x4_t{pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]), pack_bf16x2(u[4], u[5]),
                      pack_bf16x2(u[6], u[7])};
        }
        *reinterpret_cast<u32x4_t *>(a.o_h + r * f + n) =
            u32x4_t{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]),
                    pack_bf16x2(hv[4], hv[5]), pack_bf16x2(hv[6], hv[7])};
      }
    }
  } else if (KIND == FWD_GU) {
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      const int q = q0 + qrow[j] + ec;
      if (q >= Me) continue;
      const int64_t r = (int64_t)seg0 + q;
#pragma unroll
      for (int i = 0; i < FP / 2; ++i) {
        const int n = p0 + prow[i] + er;   // gate feature; up feature = f + n
        if (n >= f) continue;
        float g[4], u[4], hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          g[v] = round_bf16(acc[i][j][v]);
          u[v] = round_bf16(acc[i + FP / 2][j][v]);
          hv[v] = swiglu_h(g[v], u[v]);
        }
        if (a.o_gu) {
          *reinterpret_cast<u32x2_t *>(a.o_gu + r * f2 + n) =
              u32x2_t{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
          *reinterpret_cast<u32x2_t *>(a.o_gu + r * f2 + f + n) =
              u32x2_t{pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3])};
        }
        *reinterpret_cast<u32x2_t *>(a.o_h + r * f + n) =
            u32x2_t{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
      }
    }
  } else if (KIND == FWD_DOWN || KIND == BWD_DX) {
    bf16_t *out = (KIND == FWD_DOWN) ? a.o_y : a.o_dx;
    float wj[FQ];   // combine weights of the wave's token rows, loaded up front
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      const int q = q0 + qrow[j] + ec;
      wj[j] = (KIND == FWD_DOWN && a.row_scale) ? a.row_scale[(int64_t)seg0 + (q < Me ? q : 0)] : 1.0f;
    }
    if constexpr (epi_via_lds<KIND, FP>()) {
      // 16 rows x 64 columns at a time through the wave's own LDS slot:
      // 4-column pieces in (lane (g, c): row c), 16-byte row chunks out (lane
      // l: chunk l%8 of rows l/8 and 8 + l/8), so that each store covers 8
      // token rows x 128 contiguous bytes.  (Measured on MI355X: stores of
      // 16 rows x 32 B cost these GEMMs 6-33% of their time; a register
      // exchange between lanes instead overflows their 256 registers.)
      const int rr = lane >> 3, ch = lane & 7;
#pragma unroll
      for (int j = 0; j < FQ; ++j) {
        const float w = wj[j];
        const int qa = q0 + qrow[j] + rr;
#pragma unroll
        for (int h = 0; h < FP / 4; ++h) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int i = 4 * h + ii;
            *reinterpret_cast<LDS_AS u32x2_t *>(epi + ec * kEpiPitch + (16 * ii + er) * 2) =
                u32x2_t{pack_bf16x2(w * acc[i][j][0], w * acc[i][j][1]),
                        pack_bf16x2(w * acc[i][j][2], w * acc[i][j][3])};
          }
          wait_vm_lgkm0<63>();               // the wave's writes have landed
          __builtin_amdgcn_wave_barrier();   // (and the reads stay behind them)
          const u32x4_t A = *reinterpret_cast<const LDS_AS u32x4_t *>(epi + rr * kEpiPitch + ch * 16);
          const u32x4_t B =
              *reinterpret_cast<const LDS_AS u32x4_t *>(epi + (rr + 8) * kEpiPitch + ch * 16);
          __builtin_amdgcn_wave_barrier();   // the next writes stay behind these reads
          const int n = p0 + prow[4 * h] + ch * 8;
          if (n < d) {
            if (qa < Me) *reinterpret_cast<u32x4_t *>(out + ((int64_t)seg0 + qa) * d + n) = A;
            if (qa + 8 < Me)
              *reinterpret_cast<u32x4_t *>(out + ((int64_t)seg0 + qa + 8) * d + n) = B;
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FQ; ++j) {
        const int q = q0 + qrow[j] + ec;
        if (q >= Me) continue;
        const int64_t r = (int64_t)seg0 + q;
        const float w = wj[j];
#pragma unroll
        for (int i = 0; i < FP; ++i) {
          const int n = p0 + prow[i] + er;
          if (n >= d) continue;
          *reinterpret_cast<u32x2_t *>(out + r * d + n) =
              u32x2_t{pack_bf16x2(w * acc[i][j][0], w * acc[i][j][1]),
                      pack_bf16x2(w * acc[i][j][2], w * acc[i][j][3])};
        }
      }
    }
  } else if (KIND == BWD_DH) {
    // The wave's 64 columns at once: fragments 0,1 and 2,3 trade 16-lane
    // rows (pair_rows: lane group g then holds 8 consecutive columns of its
    // row, from 8*sig(g) in each pair's 32), then the pairs trade places
    // between lanes c and c+8 of each 16-lane row (DPP row_ror:8): lane (g, c)
    // works on token rows c%8 ("A") and 8 + c%8 ("B") at columns
    // 32*(c >= 8) + 8*sig(g) .. +7, so the saved g, u are read and dGU
    // written 16 bytes per lane, each access 8 rows x 128 B (measured on
    // MI355X: the epilogue's loads and stores at 8 bytes per lane cost dH
    // 13-17% each).
    static_assert(KIND != BWD_DH || FP == 4, "the 64 columns of four fragments");
    const int nparts = a.PT * WP;
    const bool lo = ec < 8;
    const int c = p0 + prow[0] + (lo ? 0 : 32) + 8 * sig;
    const bool colok = c < f;
    const int cc = colok ? c : 0;   // columns past f read column 0, store nothing
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      // rows A and B of this lane (rows past the expert's end read row seg0
      // and store nothing) and their combine weights
      const int qa = q0 + qrow[j] + (ec & 7), qb = qa + 8;
      const bool oka = qa < Me, okb = qb < Me;
      const int64_t ra = (int64_t)seg0 + (oka ? qa : 0), rb = (int64_t)seg0 + (okb ? qb : 0);
      const float wa = a.row_scale ? a.row_scale[ra] : 1.0f;
      const float wb = a.row_scale ? a.row_scale[rb] : 1.0f;
      // the saved g, u (H is recomputed from them, bit for bit as stored)
      const u32x4_t ga = *reinterpret_cast<const u32x4_t *>(a.gu + ra * f2 + cc);
      const u32x4_t ua = *reinterpret_cast<const u32x4_t *>(a.gu + ra * f2 + f + cc);
      const u32x4_t gb = *reinterpret_cast<const u32x4_t *>(a.gu + rb * f2 + cc);
      const u32x4_t ub = *reinterpret_cast<const u32x4_t *>(a.gu + rb * f2 + f + cc);
      // Gd in the same layout
      float gda[8], gdb[8];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        uint32_t p00, p01, p10, p11;   // pair 0 (columns 0..31), pair 1 (32..63); row c
        pair_rows(__float_as_uint(acc[0][j][v]), __float_as_uint(acc[1][j][v]), p00, p01);
        pair_rows(__float_as_uint(acc[2][j][v]), __float_as_uint(acc[3][j][v]), p10, p11);
        // row_ror:8 (DPP control 0x128): lane c of each 16-lane row takes
        // lane (c + 8) % 16
        const uint32_t s00 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p00, 0x128, 0xf, 0xf, false);
        const uint32_t s01 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p01, 0x128, 0xf, 0xf, false);
        const uint32_t s10 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p10, 0x128, 0xf, 0xf, false);
        const uint32_t s11 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p11, 0x128, 0xf, 0xf, false);
        gda[v] = __uint_as_float(lo ? p00 : s10);
        gda[4 + v] = __uint_as_float(lo ? p01 : s11);
        gdb[v] = __uint_as_float(lo ? s00 : p10);
        gdb[4 + v] = __uint_as_float(lo ? s01 : p11);
      }
      float parta = 0.0f, partb = 0.0f;
#pragma unroll
      for (int half = 0; half < 2; ++half) {   // rows A, then B
        const u32x4_t gw8 = half ? gb : ga, uw8 = half ? ub : ua;
        const float w = half ? wb : wa;
        const bool ok = (half ? okb : oka) && colok;
        float dg[8], du[8], part = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint32_t gw = gw8[t >> 1], uw = uw8[t >> 1];
          const float g = bf16_bits_to_f32((t & 1) ? (gw >> 16) : (gw & 0xffffu));
          const float u = bf16_bits_to_f32((t & 1) ? (uw >> 16) : (uw & 0xffffu));
          const float gd = half ? gdb[t] : gda[t];
          const float hv = round_bf16(swiglu_h(g, u));
          const float sg = 1.0f / (1.0f + __expf(-g));
          const float silu = g * sg;
          part += ok ? hv * gd : 0.0f;
          const float dh = w * gd;
          dg[t] = dh * u * sg * (1.0f + g * (1.0f - sg));
          du[t] = dh * silu;
        }
        if (ok) {
          const int64_t r = half ? rb : ra;
          *reinterpret_cast<u32x4_t *>(a.o_dgu + r * f2 + c) =
              u32x4_t{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]),
                      pack_bf16x2(dg[4], dg[5]), pack_bf16x2(dg[6], dg[7])};
          *reinterpret_cast<u32x4_t *>(a.o_dgu + r * f2 + f + c) =
              u32x4_t{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]),
                      pack_bf16x2(du[4], du[5]), pack_bf16x2(du[6], du[7])};
        }
        if (half) partb = part; else parta = part;
      }
      // sum over the 8 lanes that share a row (fixed order: the two column
      // halves, then the 4 lane groups)
      parta += __shfl_xor(parta, 8, 64);
      partb += __shfl_xor(partb, 8, 64);
      parta += __shfl_xor(parta, 16, 64);
      partb += __shfl_xor(partb, 16, 64);
      parta += __shfl_xor(parta, 32, 64);
      partb += __shfl_xor(partb, 32, 64);
      if (a.o_drs && lane < 8) {
        if (oka) a.o_drs[ra * nparts + t.p_tile * WP + wp] = parta;
        if (okb) a.o_drs[rb * nparts + t.p_tile * WP + wp] = partb;
      }
    }
  } else {   // weight gradients: dw[e][q][p]
    const int Pdim = (KIND == BWD_DWDOWN) ? f : d;
    const int Qdim = (KIND == BWD_DWDOWN) ? d : (int)f2;
    float *out = a.o_dw + (int64_t)t.e * Pdim * Qdim;
    // The fp32 gradients are written once and not read again here: the
    // stores are non-temporal, so they do not displace the operand slabs the
    // tiles in flight share in L2 (measured: dW_down -3.5%, dW_gu -1.4%).
    // Fragments i and i+1 (P rows 16 apart) are stored together: lane
    // (g, c) of fragment i+1, rotated by 8 within its 16-lane row, trades
    // places so that one store covers Q rows c%8 with P columns 0..31 of the
    // pair (128 contiguous bytes per row) and the other store Q rows 8 + c%8.
    static_assert(FP % 2 == 0, "fragment pairs");
    const bool lo = ec < 8;
    const int qa = q0 + (ec & 7), pa = p0 + er + (lo ? 0 : 16), pb_ = p0 + er + (lo ? 16 : 0);
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      const int qA = qa + qrow[j], qB = qA + 8;
#pragma unroll
      for (int i = 0; i < FP; i += 2) {
        f32x4_t r, A, B;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // row_ror:8 (DPP control 0x128): lane c of each 16-lane row takes
          // lane (c + 8) % 16.  (The element goes through a scalar: a bit
          // cast of a vector element expression here read element 0.)
          const float e = acc[i + 1][j][v];
          r[v] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(e), 0x128, 0xf, 0xf, false));
          A[v] = lo ? acc[i][j][v] : r[v];
          B[v] = lo ? r[v] : acc[i][j][v];
        }
        const int pA = pa + prow[i], pB = pb_ + prow[i];
        if (qA < Qdim && pA < Pdim)
          __builtin_nontemporal_store(A, reinterpret_cast<f32x4_t *>(out + (int64_t)qA * Pdim + pA));
        if (qB < Qdim && pB < Pdim)
          __builtin_nontemporal_store(B, reinterpret_cast<f32x4_t *>(out + (int64_t)qB * Pdim + pB));
      }
    }
  }
}

// ------------------------------------------------------------------ kernel

// s_waitcnt for the loads of the stage that has `younger` stages of LOADS
// loads each issued after it (loads complete in issue order; stores in
// flight only make the count conservative), and for all LDS reads.
template <int LOADS>
__device__ __forceinline__ void wait_stage(int younger) {
  if (younger >= 3) wait_vm_lgkm0<3 * LOADS>();
  else if (younger == 2) wait_vm_lgkm0<2 * LOADS>();
  else if (younger == 1) wait_vm_lgkm0<LOADS>();
  else wait_vm_lgkm0<0>();
}

// Number of a wave's Q fragments (16 token rows each, from token row q)
// that hold tokens of an expert with Me rows; weight-gradient tiles are
// always whole.
template <bool WG, int FQ>
__device__ __forceinline__ int live_frags(int q, int Me) {
  if (WG) return FQ;
  const int rows = Me - q;
  return rows <= 0 ? 0 : min(FQ, (rows + 15) >> 4);
}

// acc[i][j] += P-fragment i x Q-fragment j for the live Q fragments (token
// rows past an expert's end are zeros; their products are skipped).
template <int FP, int FQ>
__device__ __forceinline__ void mfma_block(f32x4_t (&acc)[FP][FQ], const bf16x8_t (&pf)[FP],
                                           const bf16x8_t (&qf)[FQ], int nlive) {
#pragma unroll
  for (int j = 0; j < FQ; ++j) {
    if (j < nlive) {
#pragma unroll
      for (int i = 0; i < FP; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[i], qf[j], acc[i][j], 0, 0, 0);
    }
  }
}

// Persistent: the grid has one block per CU (a multiple of 8).  The logical
// tiles are split into 8 contiguous chunks, one per XCD (workgroups are dealt
// round-robin over the XCDs), and the blocks of an XCD take its chunk's tiles
// round-robin.  A block runs its tiles as one flat sequence of 32-wide K
// stages through a ring of NS LDS buffers filled by direct-to-LDS loads NS
// stages ahead, across tile boundaries.
//
// Each wave keeps the MFMA fragments of the stage it computes in registers:
// after the barrier that publishes stage n+1 (every wave's loads of it have
// landed, every wave's reads of stage n are done, so stage n's buffer takes
// the loads of stage n+NS), the wave reads stage n+1's fragments between the
// MFMAs of stage n.  After a tile's epilogue, the next tile's first MFMAs are
// issued before the wait, so the epilogue's stores drain under them.
template <int KIND, int BP, int BQ, int WP, int WQ, int NS, int BK, bool LORA = false,
          bool GATHER = false, bool EARLY = false>
__global__ __launch_bounds__(WP *WQ * 64) void k_grouped_gemm(GemmArgs a) {
  using KT = KindTraits<KIND>;
  constexpr int NW = WP * WQ;
  // gathered token rows: the Q operand of FWD_GU / BWD_DH, the P operand's
  // k-rows of BWD_DWGU
  constexpr bool GQ = GATHER && (KIND == FWD_GU || KIND == BWD_DH);
  constexpr bool GP = GATHER && KIND == BWD_DWGU;
  static_assert(!GATHER || ((GQ || GP) && !LORA), "gathered kinds");
  // EARLY: the next stage's loads are planned (resources and LDS
  // destinations, all scalar work) before the stage barrier, so that the
  // planning overlaps the other waves' last MFMAs instead of following the
  // barrier on every wave.  Only where no plan issues loads at once: the
  // host takes it for K-tail-free token GEMMs (a K tail's plan loads its
  // stage directly, as does the LoRA stage); measured on MI355X: down and
  // dX 4-6% faster, the gathered gate/up and dH GEMMs and the weight-gradient
  // GEMMs not.
  constexpr bool EARLY_PLAN = EARLY && !GQ && !GP && !LORA && !KT::WG;
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  constexpr int FP = BP / WP / 16;
  constexpr int FQ = BQ / WQ / 16;
  static_assert(FP >= 1 && FQ >= 1 && (FQ % FP == 0 || FP % FQ == 0), "fragment counts");
  // interleaved stage: the new Q fragments are read QPR per P row in the
  // first QROWS rows, the loads go out DPR per P row
  constexpr int QPR = FQ > FP ? FQ / FP : 1, QROWS = FQ > FP ? FP : FQ;
  static_assert(!KT::PAIRED || (FP % 2 == 0), "paired tiles need an even fragment count");
  static_assert(BP % 128 == 0 && BQ % 128 == 0, "tiles are multiples of 128 rows");
  static_assert(BK == 32 || BK == 64, "stages of one or two 32-wide k steps");
  constexpr int KS = BK / 32;                                // k steps per stage
  constexpr int NIP = BP * BK / 512 / NW, NIQ = BQ * BK / 512 / NW;
  // direct loads per thread per stage (GP: one more, the token indices of
  // the stage NS ahead)
  constexpr int LOADS = NIP + NIQ + (GP ? 1 : 0);
  constexpr int SP = BP * BK / 8, SS = (BP + BQ) * BK / 8;   // 16-byte slots: P part, stage
  static_assert(NS >= 2 && NS <= 4, "two to four LDS stages");
  static_assert(3 * LOADS < 64, "vmcnt range");
  constexpr int DPR = (LOADS + FP - 1) / FP;
  constexpr int RP = KT::PT_ ? 2 : 1, RQ = KT::QT_ ? 2 : 1;  // LDS reads per fragment

  __shared__ u32x4_t smem[NS * SS];
  __shared__ int s_off[kMaxExperts + 1], s_ts[kMaxExperts + 1];
  __shared__ u32x4_t sdummy[64];   // target of loads that read nothing
  __shared__ int s_ring[16];       // token GEMMs: the block's tile sequence
  // GP: per wave, a ring of 8 entries of 64 top-k slot indices (the wave's
  // k-rows of one stage in the first KRW)
  __shared__ int s_gidx[GP ? NW * 8 * 64 : 1];
  // the epilogue's per-wave slots (down and dX GEMMs of 128 x 64 waves)
  __shared__ u32x4_t sepi[epi_via_lds<KIND, FP>() ? NW * kEpiSlot / 16 : 1];
  const LDS_AS char *lds = (const LDS_AS char *)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wp = wave % WP, wq = wave / WP;
  LDS_AS char *const epi = (LDS_AS char *)sepi + (epi_via_lds<KIND, FP>() ? wave * kEpiSlot : 0);

  const int per = gridDim.x >> 3;                  // blocks per XCD
  // Token GEMMs: tiles differ in cost (an expert's last token tile is
  // partly empty), so after its first tile a block takes the next free tile
  // of its XCD's chunk from that XCD's counter.  The block's sequence of
  // tiles goes through the LDS ring s_ring: wave 0 fetches tile number
  // n + NS of the sequence when the loads reach tile n, at least one
  // barrier before any wave needs it.  Weight-gradient tiles all cost the
  // same per expert: blocks take them round-robin.
  int total = 0;
  if (KT::WG) {
    total = a.nlogical;
  } else {
    total = a.tile_start[a.E];
  }
  total = __builtin_amdgcn_readfirstlane(total);
  // Token tiles cost about the same: equal counts per XCD.  A weight-gradient
  // tile costs its expert's M_e K rows, so those chunks come cost-balanced
  // from k_wg_bounds.
  const int chunk = (total + 7) >> 3;
  int cbeg = (blockIdx.x & 7) * chunk;
  int cend = min(total, cbeg + chunk);
  if (KT::WG && a.wg_bounds) {
    cbeg = __builtin_amdgcn_readfirstlane(a.wg_bounds[blockIdx.x & 7]);
    cend = __builtin_amdgcn_readfirstlane(a.wg_bounds[(blockIdx.x & 7) + 1]);
  }
  const int first = cbeg + (blockIdx.x >> 3);
  int32_t *const ctr = KT::WG ? nullptr : a.counters + (blockIdx.x & 7);
#define MOE_FETCH() ({                                                                        \
    const int t_ = cbeg + per + atomicAdd(ctr, 1);                                            \
    t_ < cend ? t_ : -1;                                                                      \
  })

  // routing maps into LDS: tile decodes then never wait on vector memory
  for (int i = tid; i <= a.E; i += NW * 64) {
    s_off[i] = a.offsets[i];
    if (!KT::WG) s_ts[i] = a.tile_start[i];
  }
  if (!KT::WG && tid == 0) {
    s_ring[0] = first < cend ? first : -1;
    for (int n = 1; n <= NS; ++n) s_ring[n] = first < cend ? MOE_FETCH() : -1;
  }
  __syncthreads();

  // fragment rows inside the LDS tiles (fixed per wave)
  const int prow0 = KT::PAIRED ? wp * (BP / 2 / WP) : wp * (BP / WP);
  const int qrow0 = wq * (BQ / WQ);
  int prow[FP], qrow[FQ];
#pragma unroll
  for (int i = 0; i < FP; ++i) prow[i] = prow0 + frag_delta<KT::PAIRED, BP, FP>(i);
#pragma unroll
  for (int j = 0; j < FQ; ++j) qrow[j] = qrow0 + 16 * j;

  // loop-invariant load and read offsets
  const int d = a.d, f = a.f;
  const int pld = (KIND == FWD_GU || KIND == BWD_DX || KIND == BWD_DWGU) ? d : f;
  const int qld = (KIND == FWD_DOWN) ? f : (KIND == BWD_DX || KIND == BWD_DWGU) ? 2 * f : d;
  uint32_t voffP[NIP < 2 ? NIP : 2], voffQ[NIQ < 2 ? NIQ : 2], vstrP, vstrQ;
  init_voff<BP, KT::PT_, KT::PAIRED, NW, BK>(pld, wave, lane, voffP, vstrP);
  init_voff<BQ, KT::QT_, false, NW, BK>(qld, wave, lane, voffQ, vstrQ);
  // gathered operands: offsets per tile (GQ) or per stage (GP)
  uint32_t gvoffQ[GQ ? NIQ : 1], gvoffP[GP ? NIP : 1];
  // GP: the wave's NIP loads of a transposed stage cover KRW k-rows
  constexpr int C16P = BP / 8, KRW = GP ? NIP * 64 / C16P : 1;
  static_assert(!GP || (64 % C16P == 0 && KRW <= 64), "k-rows per wave");
  const uint32_t xoff = lane < KRW ? (uint32_t)(KRW * wave + lane) * 4u : kOOB;
  uint32_t rdP[KT::PT_ ? FP : KS], rdQ[KT::QT_ ? FQ : KS];
  if constexpr (KT::PT_) {
#pragma unroll
    for (int i = 0; i < FP; ++i) rdP[i] = tr_frag_off<BP>(prow[i], lane);
  } else {
#pragma unroll
    for (int h = 0; h < KS; ++h) rdP[h] = kc_frag_off<BK>(prow0, h, lane);
  }
  if constexpr (KT::QT_) {
#pragma unroll
    for (int j = 0; j < FQ; ++j) rdQ[j] = (uint32_t)(SP * 16) + tr_frag_off<BQ>(qrow[j], lane);
  } else {
#pragma unroll
    for (int h = 0; h < KS; ++h) rdQ[h] = (uint32_t)(SP * 16) + kc_frag_off<BK>(qrow0, h, lane);
  }

  f32x4_t acc[FP][FQ];
#pragma unroll
  for (int i = 0; i < FP; ++i)
#pragma unroll
    for (int j = 0; j < FQ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // ---- issue cursor: next stage to load
  int iL = first, ikt = 0, iseq = 0;
  bool ivalid = iL < cend;
  Tile it{};
  if (ivalid) it = make_tile<KIND, BP, BQ, BK, LORA>(a, s_off, s_ts, iL);
  while (ivalid && it.nk == 0) {
    iL += per;
    ivalid = iL < cend;
    if (ivalid) it = make_tile<KIND, BP, BQ, BK, LORA>(a, s_off, s_ts, iL);
  }
  if constexpr (GQ) {
    if (ivalid) gather_rows_voff<BQ, NW, BK>(a, it.seg0, it.q0, it.Me, qld, wave, lane, gvoffQ);
  }
  int s_issued = 0, s_done = 0;

  // GP index cursor: the stage NS ahead of the issue cursor (same tile walk);
  // its top-k slots go into the wave's ring entry (stage % 8) with the loads
  // of the stage NS before it, so they have landed when that stage is planned.
  int xL = iL, xkt = 0, xseg0 = 0, xMe = 0, xnk = 0;
  bool xvalid = ivalid;
  if (GP && xvalid) { xseg0 = it.seg0; xMe = it.Me; xnk = it.nk; }
  u32x4_t rsX = make_rsrc(a.offsets, 0);
  uint32_t mX = 0;
#define MOE_XPLAN(stage)                                                                      \
  do {                                                                                        \
    rsX = xvalid ? make_rsrc(a.row_to_slot + xseg0 + xkt * BK,                                \
                             (uint32_t)max(0, xMe - xkt * BK) * 4u)                           \
                 : make_rsrc(a.offsets, 0);                                                   \
    mX = lds_addr(s_gidx + (wave * 8 + ((stage) & 7)) * 64);                                  \
    if (xvalid && ++xkt >= xnk) {                                                             \
      xkt = 0;                                                                                \
      do {                                                                                    \
        xL += per;                                                                            \
        xvalid = xL < cend;                                                                   \
        if (xvalid) {                                                                         \
          const int xe_ = xL / (a.PT * a.QT);                                                 \
          xseg0 = __builtin_amdgcn_readfirstlane(s_off[xe_]);                                 \
          xMe = __builtin_amdgcn_readfirstlane(s_off[xe_ + 1]) - xseg0;                       \
          xnk = (xMe + BK - 1) / BK;                                                          \
        }                                                                                     \
      } while (xvalid && xnk == 0);                                                           \
    }                                                                                         \
  } while (0)
  // GP: the top-k slots of the stage to plan next (read one plan ahead)
  int nslot[GP ? NIP : 1] = {};
  if constexpr (GP) {
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      MOE_XPLAN(n);
      dma4_at(rsX, mX, xoff);
    }
    wait_vm_lgkm0<0>();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NIP; ++i)
      nslot[i] = s_gidx[wave * 8 * 64 + ((wave * NIP + i) * 64 + lane) / C16P - KRW * wave];
  }

  // Loads of stage s_issued: planned once per stage (resources and LDS
  // destinations in scalar registers), issued one instruction at a time,
  // then the cursor moves on.  With every stage issued, planned loads read
  // nothing into the spare slot.
  const uint32_t dummy = lds_addr(sdummy);
  u32x4_t rsP = make_rsrc(a.offsets, 0), rsQ = rsP;
  uint32_t mP = dummy, mQ = dummy, stepP = 0, stepQ = 0;
#define MOE_PLAN()                                                                            \
  do {                                                                                        \
    if (ivalid && LORA && ikt == it.nk - 1) {                                                 \
      /* the LoRA stage: both operands through the general path, K = lora_r */                \
      u32x4_t *st_ = smem + ((unsigned)s_issued % NS) * SS;                                   \
      issue_stage<BP, KT::PT_, KT::PAIRED, NW, BK>(it.lpb, it.lpb2, it.lpld, it.prv,          \
                                                   a.lora_r, 0, st_, wave, lane);             \
      issue_stage<BQ, KT::QT_, false, NW, BK>(it.lqb, it.lqb, a.lora_r, it.qrv, a.lora_r, 0,  \
                                              st_ + SP, wave, lane);                          \
      rsP = make_rsrc(a.offsets, 0);                                                          \
      rsQ = rsP;                                                                              \
      mP = mQ = dummy;                                                                        \
      stepP = stepQ = 0;                                                                      \
    } else if (ivalid) {                                                                      \
      u32x4_t *st_ = smem + ((unsigned)s_issued % NS) * SS;                                   \
      if constexpr (GP) {                                                                     \
        MOE_GPLAN_P(st_);                                                                     \
      } else {                                                                                \
        plan_operand<BP, KT::PT_, KT::PAIRED, NW, BK>(it.pb, it.pb2, pld, it.prv, it.pkv,     \
                                                      ikt * BK, st_, wave, lane, dummy, rsP,  \
                                                      mP, stepP);                             \
      }                                                                                       \
      if constexpr (GQ) {                                                                     \
        plan_gather_rows<BQ, NW, BK>(a, qld, it.qkv, ikt * BK, st_ + SP, wave, lane, dummy,   \
                                     gvoffQ, rsQ, mQ, stepQ);                                 \
      } else {                                                                                \
        plan_operand<BQ, KT::QT_, false, NW, BK>(it.qb, it.qb, qld, it.qrv, it.qkv, ikt * BK, \
                                                 st_ + SP, wave, lane, dummy, rsQ, mQ,        \
                                                 stepQ);                                      \
      }                                                                                       \
    } else {                                                                                  \
      rsP = make_rsrc(a.offsets, 0);                                                          \
      rsQ = rsP;                                                                              \
      mP = mQ = dummy;                                                                        \
      stepP = stepQ = 0;                                                                      \
    }                                                                                         \
    if constexpr (GP) {                                                                       \
      MOE_XPLAN(s_issued + NS);                                                               \
      if (!ivalid) mX = dummy;                                                                \
    }                                                                                         \
  } while (0)
#define MOE_DMA(n)                                                                            \
  do {                                                                                        \
    if ((n) < NIP) {                                                                          \
      if constexpr (GP)                                                                       \
        dma16_at(rsP, mP + (n) * stepP, gvoffP[GP ? (n) : 0]);                                \
      else                                                                                    \
        dma16_at(rsP, mP + (n) * stepP, voffP[(n) % 2] + ((n) / 2) * vstrP);                  \
    } else if ((n) < NIP + NIQ) {                                                             \
      if constexpr (GQ)                                                                       \
        dma16_at(rsQ, mQ + ((n) - NIP) * stepQ, gvoffQ[GQ ? (n) - NIP : 0]);                  \
      else                                                                                    \
        dma16_at(rsQ, mQ + ((n) - NIP) * stepQ,                                               \
                 voffQ[((n) - NIP) % 2] + (((n) - NIP) / 2) * vstrQ);                         \
    } else {                                                                                  \
      dma4_at(rsX, mX, xoff);                                                                 \
    }                                                                                         \
  } while (0)
// GP: this stage's X k-rows from the top-k slots read from the wave's ring
// at the previous plan (entries land with the loads of the stage NS before
// theirs, so the entry of the next stage is complete after this stage's
// wait); k-rows past the expert's rows read nothing.  The resource starts at
// the tile's first column: columns past d read the next token row (feeding
// only masked outputs) or zeros.
#define MOE_GPLAN_P(st_)                                                                      \
  do {                                                                                        \
    asm volatile("" ::: "memory");                                                            \
    const int k0_ = ikt * BK;                                                                 \
    const int *ent_ = s_gidx + (wave * 8 + ((s_issued + 1) & 7)) * 64;                        \
    _Pragma("unroll") for (int i = 0; i < (GP ? NIP : 0); ++i) {                              \
      const int lin_ = (wave * NIP + i) * 64 + lane;                                          \
      const int kr_ = lin_ / C16P;                                                            \
      const int c16_ = (lin_ % C16P) ^ (tr_swz(kr_) << 1);                                    \
      gvoffP[GP ? i : 0] = k0_ + kr_ < it.Me ? (slot_token(nslot[GP ? i : 0], a.kmagic) *     \
                                                    (uint32_t)pld +                           \
                                                (uint32_t)c16_ * 8u) * 2u                     \
                                             : kOOB;                                          \
      nslot[GP ? i : 0] = ent_[kr_ - KRW * wave];                                             \
    }                                                                                         \
    rsP = make_rsrc(a.gx + it.p0, (uint32_t)((a.gx_rows * pld - it.p0) * 2));                 \
    mP = lds_addr((st_) + wave * NIP * 64);                                                   \
    stepP = 1024;                                                                             \
  } while (0)
#define MOE_ADVANCE()                                                                         \
  do {                                                                                        \
    if (ivalid) {                                                                             \
      ++s_issued;                                                                             \
      if (++ikt >= it.nk) {                                                                   \
        ikt = 0;                                                                              \
        if (KT::WG) {                                                                         \
          do {                                                                                \
            iL += per;                                                                        \
            ivalid = iL < cend;                                                               \
            if (ivalid) it = make_tile<KIND, BP, BQ, BK, LORA>(a, s_off, s_ts, iL);                 \
          } while (ivalid && it.nk == 0);                                                     \
        } else {                                                                              \
          ++iseq;                                                                             \
          iL = __builtin_amdgcn_readfirstlane(s_ring[iseq & 15]);                             \
          ivalid = iL >= 0;                                                                   \
          if (ivalid) {                                                                       \
            it = make_tile<KIND, BP, BQ, BK, LORA>(a, s_off, s_ts, iL);                             \
            if (tid == 0) s_ring[(iseq + NS) & 15] = MOE_FETCH();                             \
            if constexpr (GQ)                                                                 \
              gather_rows_voff<BQ, NW, BK>(a, it.seg0, it.q0, it.Me, qld, wave, lane,         \
                                           gvoffQ);                                           \
          }                                                                                   \
        }                                                                                     \
      }                                                                                       \
    }                                                                                         \
  } while (0)
// Stage barrier and the plan of the next loads (EARLY_PLAN: the plan first)
#define MOE_SYNC_PLAN()                                                                       \
  do {                                                                                        \
    if constexpr (EARLY_PLAN) {                                                               \
      MOE_PLAN();                                                                             \
      MOE_SYNC();                                                                             \
    } else {                                                                                  \
      MOE_SYNC();                                                                             \
      MOE_PLAN();                                                                             \
    }                                                                                         \
  } while (0)
#define MOE_ISSUE_ALL()                                                                       \
  do {                                                                                        \
    MOE_PLAN();                                                                               \
    _Pragma("unroll") for (int n_ = 0; n_ < LOADS; ++n_) MOE_DMA(n_);                         \
    MOE_ADVANCE();                                                                            \
  } while (0)

  // prologue: the first NS stages.  GP: planning stage n reads the slot
  // entry of stage n + 1; entries 1..NS-1 came with the initial loads (waited
  // for above), entry NS with stage 0's loads, so the plan of stage NS - 1
  // first waits for stage 0 (NS - 2 younger stages in flight).  From then on
  // MOE_SYNC has stage s_done + 1 landed before stage s_done + NS is planned,
  // and that stage carried the entry the plan reads.
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    if constexpr (GP) {
      if (n == NS - 1 && ivalid) wait_stage<LOADS>(NS - 2);
    }
    if (ivalid) MOE_ISSUE_ALL();
  }

  // ---- compute cursor
  int cL = first, cseq = 0;
  bool cvalid = cL < cend;
  Tile ct{};
  if (cvalid) ct = make_tile<KIND, BP, BQ, BK, LORA>(a, s_off, s_ts, cL);
  while (cvalid && ct.nk == 0) {   // experts with no rows: zero weight gradients
    epilogue<KIND, FP, FQ, WP>(a, ct, acc, prow, qrow, lane, wp, epi);
    cL += per;
    cvalid = cL < cend;
    if (cvalid) ct = make_tile<KIND, BP, BQ, BK, LORA>(a, s_off, s_ts, cL);
  }
  // live Q fragments of this wave in the current tile (a prefix)
  int nlive = cvalid ? live_frags<KT::WG, FQ>(ct.q0 + qrow0, ct.Me) : 0;

  // All fragments of k step `half` of the stage in LDS buffer (stage % NS)
  // into registers.
#define MOE_READ_STEP(stage, half)                                                            \
  do {                                                                                        \
    const LDS_AS char *rb_ = lds + ((unsigned)(stage) % NS) * (SS * 16);                      \
    _Pragma("unroll") for (int i = 0; i < FP; ++i)                                            \
        pf[i] = frag_at<KT::PT_, KT::PAIRED, BP, BK, FP>(rb_, rdP, i, (half));                \
    _Pragma("unroll") for (int j = 0; j < FQ; ++j)                                            \
        qf[j] = frag_at<KT::QT_, false, BQ, BK, FQ>(rb_, rdQ, j, (half));                     \
  } while (0)

  // MFMAs of the fragments in registers with the fragments of k step rh of
  // stage rs read in between: after P-fragment i's MFMAs its register takes
  // the new P-fragment i; the new Q-fragments arrive in spare registers
  // during the first FQ rows.  With LD, the loads planned by MOE_PLAN go out
  // one per P-fragment row.
#define MOE_WARM(rs, rh, LD)                                                                  \
  do {                                                                                        \
    const LDS_AS char *nb_ = lds + ((unsigned)(rs) % NS) * (SS * 16);                         \
    bf16x8_t qn_[FQ];                                                                         \
    _Pragma("unroll") for (int i = 0; i < QROWS; ++i) {                                       \
      _Pragma("unroll") for (int j = 0; j < FQ; ++j)                                          \
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[i], qf[j], acc[i][j], 0, 0, 0); \
      pf[i] = frag_at<KT::PT_, KT::PAIRED, BP, BK, FP>(nb_, rdP, i, (rh));                    \
      _Pragma("unroll") for (int r = 0; r < QPR; ++r)                                         \
          qn_[i * QPR + r] = frag_at<KT::QT_, false, BQ, BK, FQ>(nb_, rdQ, i * QPR + r, (rh)); \
      __builtin_amdgcn_sched_group_barrier(0x008, FQ, 0);                                     \
      __builtin_amdgcn_sched_group_barrier(0x100, RP + QPR * RQ, 0);                          \
      if (LD) { _Pragma("unroll") for (int r = 0; r < DPR; ++r)                               \
          if (i * DPR + r < LOADS) MOE_DMA(i * DPR + r); }                                    \
    }                                                                                         \
    _Pragma("unroll") for (int i = QROWS; i < FP; ++i) {                                      \
      _Pragma("unroll") for (int j = 0; j < FQ; ++j)                                          \
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[i], qf[j], acc[i][j], 0, 0, 0); \
      pf[i] = frag_at<KT::PT_, KT::PAIRED, BP, BK, FP>(nb_, rdP, i, (rh));                    \
      __builtin_amdgcn_sched_group_barrier(0x008, FQ, 0);                                     \
      __builtin_amdgcn_sched_group_barrier(0x100, RP, 0);                                     \
      if (LD) { _Pragma("unroll") for (int r = 0; r < DPR; ++r)                               \
          if (i * DPR + r < LOADS) MOE_DMA(i * DPR + r); }                                    \
    }                                                                                         \
    _Pragma("unroll") for (int j = 0; j < FQ; ++j) qf[j] = qn_[j];                            \
  } while (0)

  // Wait until stage s_done + 1 has landed and every wave is done reading
  // stage s_done; stage s_done's buffer then takes the next loads.
#define MOE_SYNC()                                                                            \
  do {                                                                                        \
    const bool has_next_ = s_done + 1 < s_issued;                                             \
    wait_stage<LOADS>(has_next_ ? s_issued - s_done - 2 : 0);                                 \
    __builtin_amdgcn_s_barrier();                                                             \
  } while (0)

  bf16x8_t pf[FP], qf[FQ];
  if (cvalid) {
    wait_stage<LOADS>(s_issued - 1);
    __builtin_amdgcn_s_barrier();
    MOE_READ_STEP(0, 0);
  }

  // One tile per pass; the fragments of its first k step are in registers.
  // Each stage holds KS k steps of 32; the barrier that publishes stage n+1
  // (and frees stage n's buffer for the loads of stage n + NS) comes before
  // the last k step of stage n.  A tile's first and last k steps issue their
  // MFMAs before that wait (the first ones overlap the previous tile's
  // stores); in between, whole tiles read the next k step between the MFMAs,
  // and tiles with token rows missing read it after them.
  while (cvalid) {
    const int nk = ct.nk;
    if (nlive >= FQ) {
      mfma_block<FP, FQ>(acc, pf, qf, FQ);
      if constexpr (KS == 1) {
        MOE_SYNC();
        if (ivalid) MOE_ISSUE_ALL();
        if (nk > 1) MOE_READ_STEP(s_done + 1, 0);
        ++s_done;
        // two stages per pass, so that the Q fragments read during a stage's
        // MFMAs alternate between two register sets; with one stage per pass
        // the compiler copies them back, waiting for the reads, before each
        // stage's first MFMA
        int kt = 1;
        for (; kt + 1 < nk - 1; kt += 2) {
          MOE_SYNC_PLAN();
          MOE_WARM(s_done + 1, 0, true);
          MOE_ADVANCE();
          ++s_done;
          MOE_SYNC_PLAN();
          MOE_WARM(s_done + 1, 0, true);
          MOE_ADVANCE();
          ++s_done;
        }
        if (kt < nk - 1) {
          MOE_SYNC_PLAN();
          MOE_WARM(s_done + 1, 0, true);
          MOE_ADVANCE();
          ++s_done;
        }
        if (nk > 1) {
          mfma_block<FP, FQ>(acc, pf, qf, FQ);
          MOE_SYNC();
          if (ivalid) MOE_ISSUE_ALL();
          ++s_done;
        }
      } else {
        MOE_READ_STEP(s_done, 1);
        for (int kt = 0; kt < nk - 1; ++kt) {
          MOE_SYNC_PLAN();
          MOE_WARM(s_done + 1, 0, true);
          MOE_ADVANCE();
          ++s_done;
          MOE_WARM(s_done, 1, false);
        }
        mfma_block<FP, FQ>(acc, pf, qf, FQ);
        MOE_SYNC();
        if (ivalid) MOE_ISSUE_ALL();
        ++s_done;
      }
    } else {
      for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
        for (int h = 0; h < KS; ++h) {
          mfma_block<FP, FQ>(acc, pf, qf, nlive);
          if (h == KS - 1) {
            MOE_SYNC();
            if (ivalid) MOE_ISSUE_ALL();
            if (kt + 1 < nk) MOE_READ_STEP(s_done + 1, 0);
            ++s_done;
          } else {
            MOE_READ_STEP(s_done, h + 1);
          }
        }
      }
    }
    // The last barrier published stage s_done: the next tile's first stage.
    epilogue<KIND, FP, FQ, WP>(a, ct, acc, prow, qrow, lane, wp, epi);
#pragma unroll
    for (int i = 0; i < FP; ++i)
#pragma unroll
      for (int j = 0; j < FQ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (KT::WG) {
      do {
        cL += per;
        cvalid = cL < cend;
        if (cvalid) {
          ct = make_tile<KIND, BP, BQ, BK, LORA>(a, s_off, s_ts, cL);
          if (ct.nk == 0) epilogue<KIND, FP, FQ, WP>(a, ct, acc, prow, qrow, lane, wp, epi);
        }
      } while (cvalid && ct.nk == 0);
    } else {
      ++cseq;
      cL = __builtin_amdgcn_readfirstlane(s_ring[cseq & 15]);
      cvalid = cL >= 0;
      if (cvalid) ct = make_tile<KIND, BP, BQ, BK, LORA>(a, s_off, s_ts, cL);
    }
    if (cvalid) {
      nlive = live_frags<KT::WG, FQ>(ct.q0 + qrow0, ct.Me);
      MOE_READ_STEP(s_done, 0);
    }
  }
#undef MOE_SYNC
#undef MOE_SYNC_PLAN
#undef MOE_READ_STEP
#undef MOE_WARM
#undef MOE_PLAN
#undef MOE_DMA
#undef MOE_ADVANCE
#undef MOE_ISSUE_ALL
#undef MOE_XPLAN
#undef MOE_GPLAN_P
#undef MOE_FETCH
}

// Threads of the one-block scans over the experts below: a power of two
// >= E, at least a wave (the scan takes log2 of it barrier rounds).
static unsigned scan_threads(int E) {
  unsigned n = 64;
  while (n < (unsigned)E) n <<= 1;
  return n;
}

// For the two token GEMMs of a pass (token-tile heights BQa, BQb; P-tile
// counts PTa, PTb): ts[e] = sum over e' < e of ceil(M_e' / BQ) * PT, and the
// 8 tile counters that follow ts[E] cleared (one block of scan_threads(E)).
__global__ __launch_bounds__(1024) void k_tile_prefix(const int32_t *__restrict__ offsets, int E,
                                                      int BQa, int PTa, int32_t *__restrict__ tsa,
                                                      int BQb, int PTb, int32_t *__restrict__ tsb) {
  __shared__ int s[1024], sb[1024];
  const int e = threadIdx.x;
  int v = 0, vb = 0;
  if (e < E) {
    const int m = offsets[e + 1] - offsets[e];
    v = (m + BQa - 1) / BQa;
    vb = (m + BQb - 1) / BQb;
  }
  s[e] = v;
  sb[e] = vb;
  __syncthreads();
  for (int off = 1; off < (int)blockDim.x; off <<= 1) {
    const int t = e >= off ? s[e - off] : 0;
    const int tb = e >= off ? sb[e - off] : 0;
    __syncthreads();
    s[e] += t;
    sb[e] += tb;
    __syncthreads();
  }
  if (e < E) {
    tsa[e + 1] = s[e] * PTa;
    tsb[e + 1] = sb[e] * PTb;
  }
  if (e == 0) tsa[0] = tsb[0] = 0;
  if (e < 8) tsa[E + 1 + e] = tsb[E + 1 + e] = 0;   // the GEMMs' per-XCD tile counters
}

// Chunk bounds of the two weight-gradient GEMMs of a backward pass (PTa x QTa
// and PTb x QTb tiles per expert, expert-major): 8 contiguous chunks of equal
// modelled cost, one per XCD.  A tile of expert e costs ceil(M_e / BK) K
// stages plus kWgTileCost stages' worth for its epilogue (an empty expert's
// tiles only store zeros).  Bounds are rounded to multiples of the blocks per
// XCD (pera, perb), which deal a chunk's tiles round-robin: when the costs
// are even, chunks then split into whole rounds as equal counts would.
// Chunk x is [bounds[x], bounds[x+1]).  One block.
constexpr int kWgTileCost = 8;
__global__ __launch_bounds__(1024) void k_wg_bounds(const int32_t *__restrict__ offsets, int E,
                                                    int BK, int na, int pera,
                                                    int32_t *__restrict__ ba, int nb, int perb,
                                                    int32_t *__restrict__ bb) {
  __shared__ long long s[1024];
  const int e = threadIdx.x;
  long long w = 0;
  if (e < E) w = (offsets[e + 1] - offsets[e] + BK - 1) / BK + kWgTileCost;
  s[e] = w;
  __syncthreads();
  for (int off = 1; off < (int)blockDim.x; off <<= 1) {   // inclusive prefix of the per-tile costs
    const long long t = e >= off ? s[e - off] : 0;
    __syncthreads();
    s[e] += t;
    __syncthreads();
  }
  // with n tiles per expert, the tiles before expert e cost n*lo and the
  // whole GEMM n*W; chunk x starts at the first tile before which the cost
  // reaches x*n*W/8: e*n + ceil((x*n*W/8 - n*lo) / w) for the expert holding
  // that point
  const long long W = s[E - 1], hi = s[e], lo = hi - w;
  if (e < E) {
#pragma unroll
    for (int x = 1; x < 8; ++x) {
      const long long ta = (long long)x * na * W / 8, tb = (long long)x * nb * W / 8;
      if ((long long)na * lo <= ta && ta < (long long)na * hi) {
        const int L = e * na + (int)((ta - (long long)na * lo + w - 1) / w);
        ba[x] = min(E * na, (L + pera / 2) / pera * pera);
      }
      if ((long long)nb * lo <= tb && tb < (long long)nb * hi) {
        const int L = e * nb + (int)((tb - (long long)nb * lo + w - 1) / w);
        bb[x] = min(E * nb, (L + perb / 2) / perb * perb);
      }
    }
  }
  if (e == 0) {
    ba[0] = bb[0] = 0;
    ba[8] = E * na;
    bb[8] = E * nb;
  }
}

// d_row_scale[r] = sum of its partials in fixed order
__global__ __launch_bounds__(256) void k_drs_reduce(const float *__restrict__ part, int nparts,
                                                    int64_t R, float *__restrict__ drs) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  const float *p = part + r * nparts;
  float s = 0.0f;
  int i = 0;
  if (nparts % 4 == 0) {   // 16-byte loads (rows then start 16-byte aligned)
    for (; i < nparts; i += 4) {
      const float4 v = *reinterpret_cast<const float4 *>(p + i);
      s += v.x;
      s += v.y;
      s += v.z;
      s += v.w;
    }
  }
  for (; i < nparts; ++i) s += p[i];
  drs[r] = s;
}

// ------------------------------------------------------------------ fp32 forward
//
// fp32 storage (no bf16 MFMA path): the same two contractions on the vector
// ALUs.  A block computes 64 expert rows x 64 output columns, 4 x 4 per
// thread, K staged through LDS 16 wide with coalesced 16-byte loads of the
// K-contiguous rows of both operands; every output is one fmaf chain over
// k = 0, 1, ... in order.  Tiles are (expert, column tile, row tile) with the
// row tiles fastest, from the tile starts of k_tile_prefix (64-row tiles).
// Used for fp32 workloads only.
constexpr int F32_BR = 64, F32_BC = 64, F32_BK = 16;

// expert e and its row-tile / column-tile of logical tile L (L < ts[E])
__device__ __forceinline__ void f32_tile(const int32_t *__restrict__ offsets,
                                         const int32_t *__restrict__ ts, int E, int L, int &e,
                                         int &seg0, int &M, int &r0, int &c_tile) {
  int lo = 0, hi = E;   // largest e with ts[e] <= L
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ts[mid] <= L) lo = mid; else hi = mid;
  }
  e = lo;
  seg0 = offsets[e];
  M = offsets[e + 1] - seg0;
  const int qt = (M + F32_BR - 1) / F32_BR;
  const int rem = L - ts[e];
  c_tile = rem / qt;
  r0 = (rem - c_tile * qt) * F32_BR;
}

// The 64 x 16 slab of rows [row0, row0 + nrows) of a [*, ld] fp32 matrix at
// column k0 into s[k][row] (rows past nrows and columns past ld read zeros).
// Row i of the slab is matrix row rowmap(i).
template <typename RowMap>
__device__ __forceinline__ void f32_stage(const float *__restrict__ m, int ld, int k0,
                                          RowMap rowmap, float (*s)[F32_BR + 4]) {
  const int t = threadIdx.x, i = t >> 2, kk = (t & 3) * 4;
  const int64_t row = rowmap(i);
  float4 v = {0.f, 0.f, 0.f, 0.f};
  if (row >= 0 && k0 + kk < ld) v = *reinterpret_cast<const float4 *>(m + row * ld + k0 + kk);
  s[kk][i] = v.x;
  s[kk + 1][i] = v.y;
  s[kk + 2][i] = v.z;
  s[kk + 3][i] = v.w;
}

// GU = [X W_g^T | X W_u^T], H = silu(g) u.  Column tile: 32 hidden units, whose
// gate and up rows of W_gu are the block's 64 columns.
__global__ __launch_bounds__(256) void k_ffn_gu_f32(const float *__restrict__ x_perm,
                                                    const int32_t *__restrict__ offsets,
                                                    const int32_t *__restrict__ ts, int E, int d,
                                                    int f, const float *__restrict__ w_gu,
                                                    float *__restrict__ gu, float *__restrict__ h) {
  __shared__ float sx[F32_BK][F32_BR + 4], sw[F32_BK][F32_BC + 4];
  const int L = blockIdx.x;
  if (L >= ts[E]) return;
  int e, seg0, M, r0, ct;
  f32_tile(offsets, ts, E, L, e, seg0, M, r0, ct);
  const int u0 = ct * (F32_BC / 2);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const auto xrow = [&](int i) -> int64_t { return r0 + i < M ? (int64_t)seg0 + r0 + i : -1; };
  const auto wrow = [&](int i) -> int64_t {   // columns 0..31 gate units, 32..63 up units
    const int u = u0 + (i & 31);
    return u < f ? (int64_t)e * 2 * f + (i < 32 ? 0 : f) + u : -1;
  };
  float acc[4][4];   // rows ty*4 + i; gate units tx*2, tx*2 + 1, then their up units
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int k0 = 0; k0 < d; k0 += F32_BK) {
    f32_stage(x_perm, d, k0, xrow, sx);
    f32_stage(w_gu, d, k0, wrow, sw);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < F32_BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sx[kk][ty * 4 + i];
      b[0] = sw[kk][tx * 2];
      b[1] = sw[kk][tx * 2 + 1];
      b[2] = sw[kk][32 + tx * 2];
      b[3] = sw[kk][32 + tx * 2 + 1];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = r0 + ty * 4 + i;
    if (rr >= M) continue;
    const int64_t r = (int64_t)seg0 + rr;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int u = u0 + tx * 2 + v;
      if (u >= f) continue;
      const float g = acc[i][v], up = acc[i][2 + v];
      if (gu) {
        gu[r * 2 * f + u] = g;
        gu[r * 2 * f + f + u] = up;
      }
      h[r * f + u] = g / (1.0f + expf(-g)) * up;
    }
  }
}

// Y_perm = w * (H W_down^T), 64 rows x 64 of the d output columns per block.
__global__ __launch_bounds__(256) void k_ffn_down_f32(const float *__restrict__ h,
                                                      const int32_t *__restrict__ offsets,
                                                      const int32_t *__restrict__ ts, int E, int d,
                                                      int f, const float *__restrict__ w_down,
                                                      const float *__restrict__ row_scale,
                                                      float *__restrict__ y) {
  __shared__ float sx[F32_BK][F32_BR + 4], sw[F32_BK][F32_BC + 4];
  const int L = blockIdx.x;
  if (L >= ts[E]) return;
  int e, seg0, M, r0, ct;
  f32_tile(offsets, ts, E, L, e, seg0, M, r0, ct);
  const int n0 = ct * F32_BC;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const auto hrow = [&](int i) -> int64_t { return r0 + i < M ? (int64_t)seg0 + r0 + i : -1; };
  const auto wrow = [&](int i) -> int64_t {
    return n0 + i < d ? (int64_t)e * d + n0 + i : -1;
  };
  float acc[4][4];   // rows ty*4 + i, columns tx*4 + j
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int k0 = 0; k0 < f; k0 += F32_BK) {
    f32_stage(h, f, k0, hrow, sx);
    f32_stage(w_down, f, k0, wrow, sw);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < F32_BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sx[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sw[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = r0 + ty * 4 + i;
    if (rr >= M) continue;
    const int64_t r = (int64_t)seg0 + rr;
    const float w = row_scale ? row_scale[r] : 1.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < d) y[r * d + n] = w * acc[i][j];
    }
  }
}

// ------------------------------------------------------------------ grouped LoRA
//
// Rank-r products of the LoRA factors over the rows of each expert (r a
// multiple of 16, at most 64).  The K-wide contractions of the block itself
// run in the grouped GEMMs above as one more K stage; these kernels form the
// r-wide operands and the factor gradients.

constexpr int kLoraMaxRank = 64;

// out[row, i] = store(s * sum_c in[row, c] * F[e][i][c]) for the rows of each
// expert e (F: [E, r, K], K contiguous); with w_out also
// out_w[row, i] = store(w[row] * out[row, i]).  One block (4 waves) per tile
// of 16 rows of one expert; wave w takes the 32-wide k steps w, w+4, ...;
// MFMA operands straight from global memory (16 bytes per lane); the four
// partial 16 x r tiles are summed in wave order through LDS.
template <int R>
__global__ __launch_bounds__(256) void k_lora_proj(const bf16_t *__restrict__ in,
                                                   const bf16_t *__restrict__ F,
                                                   const int32_t *__restrict__ offsets,
                                                   const int32_t *__restrict__ ts, int E, int K,
                                                   float scale, const float *__restrict__ w,
                                                   bf16_t *__restrict__ out,
                                                   bf16_t *__restrict__ out_w) {
  constexpr int NR = R / 16;
  __shared__ float red[4][16][R];
  const int tile = blockIdx.x;
  if (tile >= ts[E]) return;
  int lo = 0, hi = E;   // largest e with ts[e] <= tile
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ts[mid] <= tile) lo = mid; else hi = mid;
  }
  const int e = __builtin_amdgcn_readfirstlane(lo);
  const int seg0 = offsets[e], Me = offsets[e + 1] - seg0;
  const int r0 = __builtin_amdgcn_readfirstlane((tile - ts[e]) * 16);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = lane & 15, ch = lane >> 4;
  const bool rvalid = r0 + rr < Me;
  const bf16_t *arow = in + ((int64_t)seg0 + r0 + (rvalid ? rr : 0)) * K + ch * 8;
  const bf16_t *Fe = F + (int64_t)e * R * K + (int64_t)rr * K + ch * 8;
  f32x4_t acc[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  const int nsteps = (K + 31) / 32;
  constexpr int U = NR == 1 ? 16 : 8;   // steps in flight per wave
  // every pass issues the loads of U steps (steps past the end load zeros),
  // so the last, partial pass keeps its loads in flight together too
  for (int st = wave; st < nsteps; st += 4 * U) {
    u32x4_t av[U], bv[U][NR];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (st + 4 * u) * 32 + ch * 8;
      const bool kv = k < K;   // also false for steps past the end (K <= 32 * nsteps)
      av[u] = (rvalid && kv) ? *reinterpret_cast<const u32x4_t *>(arow + (st + 4 * u) * 32) : zero;
#pragma unroll
      for (int j = 0; j < NR; ++j)
        bv[u][j] = kv ? *reinterpret_cast<const u32x4_t *>(Fe + (int64_t)j * 16 * K + (st + 4 * u) * 32)
                      : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NR; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[u]), as_bf16x8(bv[u][j]),
                                                         acc[j], 0, 0, 0);
  }
  // lane holds rows 4*(lane/16) + v, rank 16*j + lane%16
#pragma unroll
  for (int j = 0; j < NR; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * ch + v][16 * j + rr] = acc[j][v];
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * R; i += 256) {
    const int row = i / R, rank = i % R;
    if (r0 + row >= Me) continue;
    const float v = ((red[0][row][rank] + red[1][row][rank]) + red[2][row][rank]) + red[3][row][rank];
    const int64_t o = ((int64_t)seg0 + r0 + row) * R + rank;
    const float z = round_bf16(scale * v);
    out[o] = (bf16_t)f32_to_bf16_bits(z);
    if (out_w) out_w[o] = (bf16_t)f32_to_bf16_bits(w[seg0 + r0 + row] * z);
  }
}

// Ft[e][i][c] = F[e][c][i]  (F: [E, K, r] -> Ft: [E, r, K]).  One block per
// (expert, 256 K-rows): the 256 x r slab is read row by row (coalesced) into
// LDS and written rank by rank (coalesced).
__global__ __launch_bounds__(256) void k_lora_transpose(const bf16_t *__restrict__ F, int E, int K,
                                                        int r, bf16_t *__restrict__ Ft) {
  __shared__ bf16_t t[256 * (kLoraMaxRank + 2)];
  const int nblk = (K + 255) / 256;
  const int e = blockIdx.x / nblk;
  const int c0 = (blockIdx.x - e * nblk) * 256;
  const int rows = min(256, K - c0);
  const int ld = r + 2;   // odd word stride: the column reads spread over the banks
  const bf16_t *src = F + ((int64_t)e * K + c0) * r;
  for (int i = threadIdx.x; i < rows * r; i += 256) t[(i / r) * ld + i % r] = src[i];
  __syncthreads();
  bf16_t *dst = Ft + (int64_t)e * r * K + c0;
  for (int i = threadIdx.x; i < rows * r; i += 256) {
    const int rank = i / rows, c = i - rank * rows;
    dst[(int64_t)rank * K + c] = t[c * ld + rank];
  }
}

// LoRA factor gradient of expert e over its rows:
//   G[c][i] = sum_{rows of e} M[row][c] * Z[row][i]     (M: [R, K], Z: [R, r])
// stored as out[e][c][i] (KR) or out[e][i][c] (RK), fp32.  One block (4
// waves) per (expert, 256-column slab of M); the rows of the expert are the
// reduction, 64 per stage, both operands staged transposed into LDS by the
// same direct loads as the weight-gradient GEMMs (Z padded to 128 columns,
// the narrowest width whose transposed layout keeps the block swizzle inside
// a k-row; columns past r are loaded but never used), three stages, two in
// flight.  Wave w owns columns 64w .. 64w+63 of the slab: 4 x (r/16) MFMA
// tiles.  Empty experts store zeros.
template <int R, bool KR>
__global__ __launch_bounds__(256) void k_lora_grad(const bf16_t *__restrict__ M,
                                                   const bf16_t *__restrict__ Z,
                                                   const int32_t *__restrict__ offsets, int E,
                                                   int K, float *__restrict__ out) {
  constexpr int BP = 256, BQ = 128, BK = 64, NW = 4, NS = 3;
  constexpr int NR = R / 16;
  constexpr int SP = BP * BK / 8, SS = (BP + BQ) * BK / 8;
  constexpr int LOADS = BP * BK / 512 / NW + BQ * BK / 512 / NW;
  __shared__ u32x4_t smem[NS * SS];
  const LDS_AS char *lds = (const LDS_AS char *)smem;
  const int nslab = (K + BP - 1) / BP;
  const int e = blockIdx.x / nslab;
  const int c0 = (blockIdx.x - e * nslab) * BP;
  const int seg0 = offsets[e], Me = offsets[e + 1] - seg0;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  uint32_t rdP[4], rdQ[NR];
#pragma unroll
  for (int i = 0; i < 4; ++i) rdP[i] = tr_frag_off<BP>(wave * 64 + 16 * i, lane);
#pragma unroll
  for (int j = 0; j < NR; ++j) rdQ[j] = (uint32_t)(SP * 16) + tr_frag_off<BQ>(16 * j, lane);
  f32x4_t acc[4][NR];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NR; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bf16_t *mb = M + (int64_t)seg0 * K + c0;
  const bf16_t *zb = Z + (int64_t)seg0 * R;
  const int nk = (Me + BK - 1) / BK;
  auto issue = [&](int kt) {
    u32x4_t *st = smem + (kt % NS) * SS;
    issue_stage<BP, true, false, NW, BK>(mb, mb, K, K - c0, Me, kt * BK, st, wave, lane);
    issue_stage<BQ, true, false, NW, BK>(zb, zb, R, R, Me, kt * BK, st + SP, wave, lane);
  };
  for (int kt = 0; kt < NS - 1 && kt < nk; ++kt) issue(kt);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + NS - 1 < nk) issue(kt + NS - 1);   // into the buffer of stage kt - 1
    const int younger = min(nk - 1 - kt, NS - 1);
    static_assert(NS - 1 <= 2 && 2 * LOADS < 64, "waits cover two younger stages");
    if (younger == 2) wait_vm_lgkm0<2 * LOADS>();
    else if (younger == 1) wait_vm_lgkm0<LOADS>();
    else wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();   // stage kt landed for every wave
    const LDS_AS char *sb = lds + (kt % NS) * (SS * 16);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8_t pf[4], qf[NR];
#pragma unroll
      for (int i = 0; i < 4; ++i) pf[i] = frag_at<true, false, BP, BK, 4>(sb, rdP, i, ks);
#pragma unroll
      for (int j = 0; j < NR; ++j) qf[j] = frag_at<true, false, BQ, BK, NR>(sb, rdQ, j, ks);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NR; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[i], qf[j], acc[i][j], 0, 0, 0);
    }
    wait_vm_lgkm0<63>();            // this wave's reads of stage kt are done
    __builtin_amdgcn_s_barrier();   // before its buffer takes stage kt + NS
  }
  // lane holds column c0 + 64*wave + 16*i + 4*(lane/16) + v, rank 16*j + lane%16
  float *oe = out + (int64_t)e * K * R;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NR; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int c = c0 + wave * 64 + 16 * i + 4 * (lane >> 4) + v;
        const int rank = 16 * j + (lane & 15);
        if (c < K) {
          if (KR) oe[(int64_t)c * R + rank] = acc[i][j][v];
          else oe[(int64_t)rank * K + c] = acc[i][j][v];
        }
      }
}

// ------------------------------------------------------------------ launch

// tile configurations (P x Q tile, wave grid, LDS stages, K per stage)
// Token GEMMs: 256 x 256 tiles, 8 waves of 128 x 64 (two per SIMD), two
// stages of 64; the dH GEMM 256 x 128 tiles (8 waves of 64 x 64, three
// stages of 64: twice the tiles, so a shorter tail and half the dSwiGLU
// epilogue per tile; measured 4% faster).  Weight gradients: 256 x 256,
// 8 waves of 128 x 64, four stages of 32 (three in flight).
constexpr int FWD_BP = 256, FWD_BQ = 256, FWD_WP = 2, FWD_WQ = 4, FWD_NS = 2, FWD_BK = 64;  // FWD_GU
constexpr int DN_BP = 256, DN_BQ = 256, DN_WP = 2, DN_WQ = 4, DN_NS = 2, DN_BK = 64;  // FWD_DOWN
constexpr int DX_BP = 256, DX_BQ = 256, DX_WP = 2, DX_WQ = 4, DX_NS = 2, DX_BK = 64;  // BWD_DX
constexpr int DH_BP = 256, DH_BQ = 128, DH_WP = 4, DH_WQ = 2, DH_NS = 3, DH_BK = 64;  // BWD_DH
// gathered FWD_GU: 64x64 waves leave room for the per-row token offsets
constexpr int FG_BP = 256, FG_BQ = 128, FG_WP = 4, FG_WQ = 2, FG_NS = 3, FG_BK = 64;
constexpr int WG_BP = 256, WG_BQ = 256, WG_WP = 2, WG_WQ = 4, WG_NS = 4, WG_BK = 32;  // weight grads

// S = store(w * dY_perm): the row-scaled upstream gradient of the
// down-projection weight gradient (bf16 rounding of the fp32 product).  One
// wave per row r (four per block), 16-byte chunks.
__global__ __launch_bounds__(256) void k_row_scale(const bf16_t *__restrict__ dy,
                                                   const float *__restrict__ w, int64_t R, int d,
                                                   bf16_t *__restrict__ s) {
  const int64_t r =
      (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (r >= R) return;
  const int lane = threadIdx.x & 63;
  const float wr = w ? w[r] : 1.0f;
  const u32x4_t *in = reinterpret_cast<const u32x4_t *>(dy + r * d);
  u32x4_t *out = reinterpret_cast<u32x4_t *>(s + r * d);
  const int nvec = d / 8;
  for (int c0 = 0; c0 < nvec; c0 += 256) {
    u32x4_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + j * 64 + lane;
      if (c < nvec) v[j] = in[c];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + j * 64 + lane;
      if (c >= nvec) continue;
      u32x4_t o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = pack_bf16x2(bf16_bits_to_f32(v[j][q] & 0xffffu) * wr,
                           bf16_bits_to_f32(v[j][q] >> 16) * wr);
      out[c] = o;
    }
  }
}

static inline int pad8(int64_t n) { return (int)((n + 7) / 8 * 8); }

// Persistent grid: one block per CU of the current device (a multiple of 8),
// never more blocks than tiles (rounded up to 8).
static int persistent_grid(int64_t tiles) {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  int g = cus[dev] / 8 * 8;
  if (g < 8) g = 8;
  const int64_t t = pad8(tiles < 1 ? 1 : tiles);
  return (int)(t < g ? t : g);
}

// tile starts and cleared counters of a pass's two token GEMMs (one launch)
static int launch_tile_prefix(const GemmArgs &a, int BQa, int PTa, int32_t *tsa, int BQb, int PTb,
                              int32_t *tsb, hipStream_t s) {
  MOE_LAUNCH("tile_prefix", s,
             k_tile_prefix<<<1, scan_threads(a.E), 0, s>>>(a.offsets, a.E, BQa, PTa, tsa, BQb,
                                                           PTb, tsb));
  return check_launch("tile_prefix");
}

template <int KIND, int BP, int BQ, int WP, int WQ, int NS, int BK, bool LORA = false,
          bool GATHER = false>
static int launch_token_gemm(GemmArgs a, int64_t R, int PT, int32_t *tile_start, const char *name,
                             hipStream_t s) {
  if (R == 0) return MOE_OK;
  a.PT = PT;
  a.tile_start = tile_start;   // filled by launch_tile_prefix
  a.counters = tile_start + a.E + 1;
  const int64_t bound = ((R + BQ - 1) / BQ + a.E) * (int64_t)PT;
  const int grid = persistent_grid(bound);
  // the plan-before-barrier instance where no stage has a K tail
  if constexpr (!LORA && !GATHER) {
    const int K = (KIND == FWD_DOWN) ? a.f : (KIND == BWD_DX) ? 2 * a.f : a.d;
    if (K % BK == 0) {
      MOE_LAUNCH(name, s,
                 (k_grouped_gemm<KIND, BP, BQ, WP, WQ, NS, BK, false, false, true>
                  <<<grid, WP * WQ * 64, 0, s>>>(a)));
      return check_launch(name);
    }
  }
  MOE_LAUNCH(name, s,
             (k_grouped_gemm<KIND, BP, BQ, WP, WQ, NS, BK, LORA, GATHER>
              <<<grid, WP * WQ * 64, 0, s>>>(a)));
  return check_launch(name);
}

template <int KIND, int BP, int BQ, int WP, int WQ, int NS, int BK, bool GATHER = false>
static int launch_wgrad_gemm(GemmArgs a, int Pdim, int Qdim, const char *name, hipStream_t s) {
  a.PT = (Pdim + BP - 1) / BP;
  a.QT = (Qdim + BQ - 1) / BQ;
  a.nlogical = a.E * a.PT * a.QT;
  const int grid = persistent_grid(a.nlogical);
  MOE_LAUNCH(name, s,
             (k_grouped_gemm<KIND, BP, BQ, WP, WQ, NS, BK, false, GATHER>
              <<<grid, WP * WQ * 64, 0, s>>>(a)));
  return check_launch(name);
}

}  // namespace moe

using namespace moe;

// ====================================================================== C ABI

static int check_ffn(const char *fn, int E, int64_t R, int d, int f, int dtype) {
  MOE_REQUIRE(E >= 1 && E <= kMaxExperts, MOE_ERR_UNSUPPORTED, "%s: E=%d", fn, E);
  MOE_REQUIRE(R >= 0 && R < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED, "%s: R=%lld", fn, (long long)R);
  MOE_REQUIRE(d > 0 && d % 8 == 0 && f > 0 && f % 8 == 0, MOE_ERR_UNSUPPORTED,
              "%s: d=%d f=%d must be positive multiples of 8", fn, d, f);
  MOE_REQUIRE((int64_t)d * f <= ((int64_t)1 << 30), MOE_ERR_UNSUPPORTED, "%s: d*f too large", fn);
  MOE_REQUIRE(dtype == MOE_BF16 || dtype == MOE_F32, MOE_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  return MOE_OK;
}

// tile_start[E+1] and 8 tile counters
static size_t tile_start_bytes(int E) { return align_up(sizeof(int32_t) * (size_t)(E + 1 + 8), 256); }

static size_t drs_bytes(int64_t R, int f) {
  const int nparts = (f + DH_BP - 1) / DH_BP * DH_WP;
  return align_up(sizeof(float) * (size_t)R * nparts, 256);
}

extern "C" size_t moe_grouped_ffn_workspace_size(int64_t R, int E, int d, int f, int dtype) {
  (void)dtype;
  if (R < 0 || E < 1 || f < 1 || d < 1) return 0;
  // tile prefixes, d_row_scale partials, S = w * dY_perm (bf16), the weight-
  // gradient chunk bounds
  return 2 * tile_start_bytes(E) + drs_bytes(R, f) + align_up(2 * (size_t)R * d, 256) + 256;
}

// bf16 forward: gate/up GEMM + SwiGLU, down GEMM + row scale.  gather: the
// gate/up GEMM reads its token rows from a.gx through a.row_to_slot.
static int ffn_fwd_bf16(GemmArgs a, int64_t R, void *ws, hipStream_t s, bool gather) {
  const int E = a.E, d = a.d, f = a.f;
  int32_t *ts0 = (int32_t *)ws;
  int32_t *ts1 = (int32_t *)((char *)ws + tile_start_bytes(E));
  static_assert(FG_BP == FWD_BP, "one gate/up P-tile count");
  const int pt_gu = (f + FWD_BP / 2 - 1) / (FWD_BP / 2), pt_dn = (d + DN_BP - 1) / DN_BP;
  int rc = launch_tile_prefix(a, gather ? FG_BQ : FWD_BQ, pt_gu, ts0, DN_BQ, pt_dn, ts1, s);
  if (rc) return rc;
  if (gather)
    rc = launch_token_gemm<FWD_GU, FG_BP, FG_BQ, FG_WP, FG_WQ, FG_NS, FG_BK, false, true>(
        a, R, pt_gu, ts0, "gg_fwd_gate_up_swiglu_gather", s);
  else
    rc = launch_token_gemm<FWD_GU, FWD_BP, FWD_BQ, FWD_WP, FWD_WQ, FWD_NS, FWD_BK>(
        a, R, pt_gu, ts0, "gg_fwd_gate_up_swiglu", s);
  if (rc) return rc;
  return launch_token_gemm<FWD_DOWN, DN_BP, DN_BQ, DN_WP, DN_WQ, DN_NS, DN_BK>(
      a, R, pt_dn, ts1, "gg_fwd_down_scale", s);
}

// Argument checks shared by the forward entry points (0 = go on).
static int check_ffn_fwd_args(const char *fn, const void *x_perm, const int32_t *offsets, int E,
                              int64_t R, int d, int f, const void *w_gu, const void *w_down,
                              int dtype, const void *gu, const void *h, const void *y_perm) {
  int rc = check_ffn(fn, E, R, d, f, dtype);
  if (rc) return rc;
  if (R == 0) return MOE_OK;
  MOE_REQUIRE(x_perm && offsets && w_gu && w_down && h && y_perm, MOE_ERR_INVALID_ARG,
              "%s: null pointer", fn);
  MOE_REQUIRE(aligned16(x_perm) && aligned16(w_gu) && aligned16(w_down) && aligned16(h) &&
                  aligned16(y_perm) && (!gu || aligned16(gu)),
              MOE_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
  return MOE_OK;
}

// The forward's launches on validated arguments; ws holds at least the two
// tile-start tables (2 * tile_start_bytes(E)).
static int ffn_fwd_run(const void *x_perm, const int32_t *offsets, int E, int64_t R, int d, int f,
                       const void *w_gu, const void *w_down, const float *row_scale, int dtype,
                       void *gu, void *h, void *y_perm, void *ws, hipStream_t s);

extern "C" int moe_grouped_ffn_fwd(const void *x_perm, const int32_t *offsets, int E, int64_t R,
                                   int d, int f, const void *w_gu, const void *w_down,
                                   const float *row_scale, int dtype, void *gu, void *h,
                                   void *y_perm, void *ws, size_t ws_bytes, void *stream) {
  clear_error();
  int rc = check_ffn_fwd_args("moe_grouped_ffn_fwd", x_perm, offsets, E, R, d, f, w_gu, w_down,
                              dtype, gu, h, y_perm);
  if (rc || R == 0) return rc;
  const size_t need = moe_grouped_ffn_workspace_size(R, E, d, f, dtype);
  MOE_REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE, "moe_grouped_ffn_fwd: workspace %zu < %zu",
              ws_bytes, need);
  return ffn_fwd_run(x_perm, offsets, E, R, d, f, w_gu, w_down, row_scale, dtype, gu, h, y_perm,
                     ws, (hipStream_t)stream);
}

// ------------------------------------------------------------------ allocation-free forward
//
// moe_grouped_ffn_fwd_noalloc keeps the forward's scratch -- two tile-start
// tables with their per-XCD tile counters, 2 * tile_start_bytes(E) bytes --
// in this file-scope array instead of a caller workspace.  Each device holds
// its own copy until the process ends; the host takes its device address once
// per device (hipGetSymbolAddress, on that device's first call) and passes
// that address to the kernels, never the array's name.  The tile-prefix
// kernel rewrites the tables and clears the counters at the start of every
// call, so nothing needs clearing in between; calls that overlap on one device
// share the array and race.
constexpr size_t kTileStartMax = (sizeof(int32_t) * (kMaxExperts + 1 + 8) + 255) / 256 * 256;
constexpr size_t kNoAllocScratchBytes = 2 * kTileStartMax;   // 8704 bytes
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_addr[kMaxDevices];

static int scratch_address(const char *fn, void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  MOE_REQUIRE(e == hipSuccess, MOE_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  MOE_REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_ERR_UNSUPPORTED, "%s: device %d", fn, dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    MOE_REQUIRE(e == hipSuccess && p, MOE_ERR_HIP, "%s: hipGetSymbolAddress: %s", fn,
                hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MOE_OK;
}

extern "C" int moe_grouped_ffn_fwd_noalloc(const void *x_perm, const int32_t *offsets, int E,
                                           int64_t R, int d, int f, const void *w_gu,
                                           const void *w_down, const float *row_scale, int dtype,
                                           void *gu, void *h, void *y_perm, void *stream) {
  clear_error();
  const char *fn = "moe_grouped_ffn_fwd_noalloc";
  int rc = check_ffn_fwd_args(fn, x_perm, offsets, E, R, d, f, w_gu, w_down, dtype, gu, h, y_perm);
  if (rc || R == 0) return rc;
  const size_t need = 2 * tile_start_bytes(E);
  MOE_REQUIRE(need <= kNoAllocScratchBytes, MOE_ERR_UNSUPPORTED,
              "%s: E=%d needs %zu bytes of scratch, more than the static %zu", fn, E, need,
              kNoAllocScratchBytes);
  void *ws = nullptr;
  rc = scratch_address(fn, &ws);
  if (rc) return rc;
  return ffn_fwd_run(x_perm, offsets, E, R, d, f, w_gu, w_down, row_scale, dtype, gu, h, y_perm,
                     ws, (hipStream_t)stream);
}

static int ffn_fwd_run(const void *x_perm, const int32_t *offsets, int E, int64_t R, int d, int f,
                       const void *w_gu, const void *w_down, const float *row_scale, int dtype,
                       void *gu, void *h, void *y_perm, void *ws, hipStream_t s) {
  int rc = MOE_OK;
  if (dtype == MOE_F32) {
    int32_t *ts0 = (int32_t *)ws;
    int32_t *ts1 = (int32_t *)((char *)ws + tile_start_bytes(E));
    const int ct_gu = (f + F32_BC / 2 - 1) / (F32_BC / 2), ct_dn = (d + F32_BC - 1) / F32_BC;
    const int64_t row_tiles = (R + F32_BR - 1) / F32_BR + E;   // a bound over the experts
    MOE_REQUIRE(row_tiles * (ct_gu > ct_dn ? ct_gu : ct_dn) < ((int64_t)1 << 31),
                MOE_ERR_UNSUPPORTED, "moe_grouped_ffn_fwd: fp32 problem too large");
    GemmArgs ta{};
    ta.offsets = offsets;
    ta.E = E;
    rc = launch_tile_prefix(ta, F32_BR, ct_gu, ts0, F32_BR, ct_dn, ts1, s);
    if (rc) return rc;
    MOE_LAUNCH("ffn_gu_f32", s,
               k_ffn_gu_f32<<<(unsigned)(row_tiles * ct_gu), 256, 0, s>>>(
                   (const float *)x_perm, offsets, ts0, E, d, f, (const float *)w_gu, (float *)gu,
                   (float *)h));
    rc = check_launch("moe_grouped_ffn_fwd(gu f32)");
    if (rc) return rc;
    MOE_LAUNCH("ffn_down_f32", s,
               k_ffn_down_f32<<<(unsigned)(row_tiles * ct_dn), 256, 0, s>>>(
                   (const float *)h, offsets, ts1, E, d, f, (const float *)w_down, row_scale,
                   (float *)y_perm));
    return check_launch("moe_grouped_ffn_fwd(down f32)");
  }
  GemmArgs a{};
  a.x_perm = (const bf16_t *)x_perm;
  a.w_gu = (const bf16_t *)w_gu;
  a.w_down = (const bf16_t *)w_down;
  a.h = (const bf16_t *)h;
  a.row_scale = row_scale;
  a.offsets = offsets;
  a.o_gu = (bf16_t *)gu;
  a.o_h = (bf16_t *)h;
  a.o_y = (bf16_t *)y_perm;
  a.E = E;
  a.d = d;
  a.f = f;
  return ffn_fwd_bf16(a, R, ws, s, false);
}

// bf16 backward: dH GEMM + dSwiGLU (+ d_row_scale), dX GEMM, the two
// weight-gradient GEMMs.  gdy (gathered): the dH GEMM and S read the rows of
// the unpermuted dY = gdy through a.row_to_slot, and without a.x_perm the
// dW_gu GEMM reads X = a.gx the same way.
static int ffn_bwd_bf16(GemmArgs a, int64_t R, float *dw_gu, float *dw_down, float *d_row_scale,
                        const bf16_t *gdy, const int32_t *slot_to_row, int k, void *ws,
                        hipStream_t s) {
  const int E = a.E, d = a.d, f = a.f;
  const bool gather = gdy != nullptr;
  int32_t *ts0 = (int32_t *)ws;
  int32_t *ts1 = (int32_t *)((char *)ws + tile_start_bytes(E));
  float *drs_part = (float *)((char *)ws + 2 * tile_start_bytes(E));
  bf16_t *s_perm = (bf16_t *)((char *)ws + 2 * tile_start_bytes(E) + drs_bytes(R, f));
  a.o_drs = drs_part;
  const int pt_dh = (f + DH_BP - 1) / DH_BP, pt_dx = (d + DX_BP - 1) / DX_BP;
  int rc = MOE_OK;
  if (R > 0) {
    rc = launch_tile_prefix(a, DH_BQ, pt_dh, ts0, DX_BQ, pt_dx, ts1, s);
    if (rc) return rc;
  }
  // 1. dGU (and d_row_scale partials) from dY_perm and W_down
  if (gather) {
    GemmArgs g = a;
    const bf16_t *x = a.gx;
    g.gx = gdy;
    rc = launch_token_gemm<BWD_DH, DH_BP, DH_BQ, DH_WP, DH_WQ, DH_NS, DH_BK, false, true>(
        g, R, pt_dh, ts0, "gg_bwd_dh_dswiglu_gather", s);
    a.gx = x;
  } else {
    rc = launch_token_gemm<BWD_DH, DH_BP, DH_BQ, DH_WP, DH_WQ, DH_NS, DH_BK>(a, R, pt_dh, ts0,
                                                               "gg_bwd_dh_dswiglu", s);
  }
  if (rc) return rc;
  if (d_row_scale && R > 0) {
    MOE_LAUNCH("drs_reduce", s,
               k_drs_reduce<<<(unsigned)((R + 255) / 256), 256, 0, s>>>(drs_part, pt_dh * DH_WP, R,
                                                                       d_row_scale));
    rc = check_launch("moe_grouped_ffn_bwd(drs)");
    if (rc) return rc;
  }
  // 2. dX_perm = dGU . W_gu
  rc = launch_token_gemm<BWD_DX, DX_BP, DX_BQ, DX_WP, DX_WQ, DX_NS, DX_BK>(a, R, pt_dx, ts1,
                                                             "gg_bwd_dx", s);
  if (rc) return rc;
  // 3. dW_down[e] = S^T H with S = store(w*dY_perm)   -> [E, d, f]
  if (R > 0) {
    const unsigned blocks = (unsigned)((R + 3) / 4);
    if (gather) {
      rc = launch_row_scale_scatter(gdy, slot_to_row, a.row_scale, R / k, d, k, s_perm, s);
      if (rc) return rc;
    } else
      MOE_LAUNCH("row_scale", s,
                 k_row_scale<<<blocks, 256, 0, s>>>(a.dy_perm, a.row_scale, R, d, s_perm));
    rc = check_launch("moe_grouped_ffn_bwd(row scale)");
    if (rc) return rc;
  }
  // weight-gradient chunks of equal modelled cost per XCD (skewed experts)
  int32_t *wgb = (int32_t *)((char *)s_perm + align_up(2 * (size_t)R * d, 256));
  const int pt_wd = (f + WG_BP - 1) / WG_BP, qt_wd = (d + WG_BQ - 1) / WG_BQ;
  const int pt_wg = (d + WG_BP - 1) / WG_BP, qt_wg = (2 * f + WG_BQ - 1) / WG_BQ;
  const int per_wd = persistent_grid((int64_t)E * pt_wd * qt_wd) / 8;
  const int per_wg = persistent_grid((int64_t)E * pt_wg * qt_wg) / 8;
  MOE_LAUNCH("wg_bounds", s,
             k_wg_bounds<<<1, scan_threads(E), 0, s>>>(a.offsets, E, WG_BK, pt_wd * qt_wd, per_wd, wgb,
                                            pt_wg * qt_wg, per_wg, wgb + 16));
  rc = check_launch("moe_grouped_ffn_bwd(wg bounds)");
  if (rc) return rc;
  a.s_perm = s_perm;
  a.o_dw = dw_down;
  a.wg_bounds = wgb;
  rc = launch_wgrad_gemm<BWD_DWDOWN, WG_BP, WG_BQ, WG_WP, WG_WQ, WG_NS, WG_BK>(a, f, d, "gg_bwd_dw_down", s);
  if (rc) return rc;
  // 4. dW_gu[e] = dGU^T X_perm        -> [E, 2f, d]
  a.o_dw = dw_gu;
  a.wg_bounds = wgb + 16;
  if (gather && !a.x_perm)
    return launch_wgrad_gemm<BWD_DWGU, WG_BP, WG_BQ, WG_WP, WG_WQ, WG_NS, WG_BK, true>(
        a, d, 2 * f, "gg_bwd_dw_gate_up_gather", s);
  return launch_wgrad_gemm<BWD_DWGU, WG_BP, WG_BQ, WG_WP, WG_WQ, WG_NS, WG_BK>(a, d, 2 * f, "gg_bwd_dw_gate_up",
                                                                s);
}

extern "C" int moe_grouped_ffn_bwd(const void *x_perm, const void *gu, const void *h,
                                   const int32_t *offsets, int E, int64_t R, int d, int f,
                                   const void *w_gu, const void *w_down, const float *row_scale,
                                   const void *dy_perm, int dtype, void *dgu, void *dx_perm,
                                   float *dw_gu, float *dw_down, float *d_row_scale, void *ws,
                                   size_t ws_bytes, void *stream) {
  clear_error();
  int rc = check_ffn("moe_grouped_ffn_bwd", E, R, d, f, dtype);
  if (rc) return rc;
  MOE_REQUIRE(dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "moe_grouped_ffn_bwd: needs MOE_BF16");
  MOE_REQUIRE(offsets && w_gu && w_down && dw_gu && dw_down, MOE_ERR_INVALID_ARG,
              "moe_grouped_ffn_bwd: null pointer");
  MOE_REQUIRE(R == 0 || (x_perm && gu && h && dy_perm && dgu && dx_perm), MOE_ERR_INVALID_ARG,
              "moe_grouped_ffn_bwd: null activation pointer");
  MOE_REQUIRE(aligned16(w_gu) && aligned16(w_down) && aligned16(dw_gu) && aligned16(dw_down) &&
                  (R == 0 || (aligned16(x_perm) && aligned16(gu) && aligned16(h) &&
                              aligned16(dy_perm) && aligned16(dgu) && aligned16(dx_perm))),
              MOE_ERR_INVALID_ARG, "moe_grouped_ffn_bwd: pointers must be 16-byte aligned");
  const size_t need = moe_grouped_ffn_workspace_size(R, E, d, f, dtype);
  MOE_REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE, "moe_grouped_ffn_bwd: workspace %zu < %zu",
              ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  GemmArgs a{};
  a.x_perm = (const bf16_t *)x_perm;
  a.w_gu = (const bf16_t *)w_gu;
  a.w_down = (const bf16_t *)w_down;
  a.h = (const bf16_t *)h;
  a.gu = (const bf16_t *)gu;
  a.dy_perm = (const bf16_t *)dy_perm;
  a.dgu = (const bf16_t *)dgu;
  a.row_scale = row_scale;
  a.offsets = offsets;
  a.o_dgu = (bf16_t *)dgu;
  a.o_dx = (bf16_t *)dx_perm;
  a.E = E;
  a.d = d;
  a.f = f;
  return ffn_bwd_bf16(a, R, dw_gu, dw_down, d_row_scale, nullptr, nullptr, 1, ws, s);
}

// ====================================================================== gathered rows

static int check_gather(const char *fn, int64_t T, int k, int d, const int32_t *row_to_slot) {
  MOE_REQUIRE(T >= 0 && k >= 1 && k <= 32, MOE_ERR_UNSUPPORTED, "%s: T=%lld k=%d", fn,
              (long long)T, k);
  MOE_REQUIRE(T * k < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED, "%s: T*k too large", fn);
  // byte offsets into the token-major sources and the slot -> token division
  // stay exact in 32 bits
  MOE_REQUIRE(T * (int64_t)d < ((int64_t)1 << 30), MOE_ERR_UNSUPPORTED,
              "%s: T*d = %lld must be below 2^30", fn, (long long)(T * (int64_t)d));
  MOE_REQUIRE(T * k * (int64_t)k < ((int64_t)1 << 32), MOE_ERR_UNSUPPORTED, "%s: T*k*k too large",
              fn);
  MOE_REQUIRE(T == 0 || row_to_slot, MOE_ERR_INVALID_ARG, "%s: null row_to_slot", fn);
  return MOE_OK;
}

static uint64_t slot_kmagic(int k) { return (((uint64_t)1) << 32) / (uint64_t)k + 1; }

extern "C" int moe_grouped_ffn_fwd_gather(const void *x, int64_t T, const int32_t *row_to_slot,
                                          int k, const int32_t *offsets, int E, int d, int f,
                                          const void *w_gu, const void *w_down,
                                          const float *row_scale, void *gu, void *h, void *y_perm,
                                          void *ws, size_t ws_bytes, void *stream) {
  clear_error();
  int rc = check_gather("moe_grouped_ffn_fwd_gather", T, k, d, row_to_slot);
  if (rc) return rc;
  const int64_t R = T * k;
  rc = check_ffn("moe_grouped_ffn_fwd_gather", E, R, d, f, MOE_BF16);
  if (rc) return rc;
  if (R == 0) return MOE_OK;
  MOE_REQUIRE(x && offsets && w_gu && w_down && h && y_perm, MOE_ERR_INVALID_ARG,
              "moe_grouped_ffn_fwd_gather: null pointer");
  MOE_REQUIRE(aligned16(x) && aligned16(w_gu) && aligned16(w_down) && aligned16(h) &&
                  aligned16(y_perm) && (!gu || aligned16(gu)),
              MOE_ERR_INVALID_ARG, "moe_grouped_ffn_fwd_gather: pointers must be 16-byte aligned");
  const size_t need = moe_grouped_ffn_workspace_size(R, E, d, f, MOE_BF16);
  MOE_REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE,
              "moe_grouped_ffn_fwd_gather: workspace %zu < %zu", ws_bytes, need);
  GemmArgs a{};
  a.x_perm = (const bf16_t *)x;   // placeholder: the gathered kernel reads gx
  a.gx = (const bf16_t *)x;
  a.gx_rows = T;
  a.row_to_slot = row_to_slot;
  a.kmagic = slot_kmagic(k);
  a.w_gu = (const bf16_t *)w_gu;
  a.w_down = (const bf16_t *)w_down;
  a.h = (const bf16_t *)h;
  a.row_scale = row_scale;
  a.offsets = offsets;
  a.o_gu = (bf16_t *)gu;
  a.o_h = (bf16_t *)h;
  a.o_y = (bf16_t *)y_perm;
  a.E = E;
  a.d = d;
  a.f = f;
  return ffn_fwd_bf16(a, R, ws, (hipStream_t)stream, true);
}

extern "C" int moe_grouped_ffn_bwd_gather(const void *x, const void *x_perm, const void *dy,
                                          int64_t T, const int32_t *row_to_slot,
                                          const int32_t *slot_to_row, int k, const void *gu,
                                          const void *h, const int32_t *offsets, int E, int d,
                                          int f, const void *w_gu, const void *w_down,
                                          const float *row_scale, void *dgu, void *dx_perm,
                                          float *dw_gu, float *dw_down, float *d_row_scale,
                                          void *ws, size_t ws_bytes, void *stream) {
  clear_error();
  int rc = check_gather("moe_grouped_ffn_bwd_gather", T, k, d, row_to_slot);
  if (rc) return rc;
  const int64_t R = T * k;
  rc = check_ffn("moe_grouped_ffn_bwd_gather", E, R, d, f, MOE_BF16);
  if (rc) return rc;
  MOE_REQUIRE(offsets && w_gu && w_down && dw_gu && dw_down, MOE_ERR_INVALID_ARG,
              "moe_grouped_ffn_bwd_gather: null pointer");
  MOE_REQUIRE(R == 0 || ((x || x_perm) && dy && gu && h && dgu && dx_perm && slot_to_row),
              MOE_ERR_INVALID_ARG, "moe_grouped_ffn_bwd_gather: null activation or map pointer");
  MOE_REQUIRE(aligned16(w_gu) && aligned16(w_down) && aligned16(dw_gu) && aligned16(dw_down) &&
                  (R == 0 || (aligned16(x) && aligned16(x_perm) && aligned16(dy) &&
                              aligned16(gu) && aligned16(h) && aligned16(dgu) &&
                              aligned16(dx_perm))),
              MOE_ERR_INVALID_ARG, "moe_grouped_ffn_bwd_gather: pointers must be 16-byte aligned");
  const size_t need = moe_grouped_ffn_workspace_size(R, E, d, f, MOE_BF16);
  MOE_REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE,
              "moe_grouped_ffn_bwd_gather: workspace %zu < %zu", ws_bytes, need);
  GemmArgs a{};
  a.x_perm = (const bf16_t *)x_perm;   // null: the dW_gu GEMM gathers X
  a.dy_perm = (const bf16_t *)dy;      // placeholder: the gathered kernels read dY as gx
  a.gx = (const bf16_t *)(x ? x : x_perm);
  a.gx_rows = T;
  a.row_to_slot = row_to_slot;
  a.kmagic = slot_kmagic(k);
  a.w_gu = (const bf16_t *)w_gu;
  a.w_down = (const bf16_t *)w_down;
  a.h = (const bf16_t *)h;
  a.gu = (const bf16_t *)gu;
  a.dgu = (const bf16_t *)dgu;
  a.row_scale = row_scale;
  a.offsets = offsets;
  a.o_dgu = (bf16_t *)dgu;
  a.o_dx = (bf16_t *)dx_perm;
  a.E = E;
  a.d = d;
  a.f = f;
  return ffn_bwd_bf16(a, R, dw_gu, dw_down, d_row_scale, (const bf16_t *)dy, slot_to_row, k, ws,
                      (hipStream_t)stream);
}

// ====================================================================== grouped LoRA

static int check_lora(const char *fn, int r, float scale) {
  MOE_REQUIRE(r >= 16 && r <= kLoraMaxRank && r % 16 == 0, MOE_ERR_UNSUPPORTED,
              "%s: rank %d (a multiple of 16 up to %d)", fn, r, kLoraMaxRank);
  MOE_REQUIRE(scale == scale && scale > -INFINITY && scale < INFINITY, MOE_ERR_INVALID_ARG,
              "%s: scale must be finite", fn);
  return MOE_OK;
}

// 16-row tile prefix, transposed B factors, u_dn, w*u_dn, u_gu after the
// plain grouped-FFN workspace
static size_t lora_extra_bytes(int64_t R, int E, int d, int f, int r) {
  return tile_start_bytes(E) + align_up(2 * (size_t)E * r * d, 256) +
         align_up(2 * (size_t)E * r * 2 * f, 256) + 3 * align_up(2 * (size_t)R * r, 256);
}

extern "C" size_t moe_grouped_ffn_lora_workspace_size(int64_t R, int E, int d, int f, int r) {
  if (R < 0 || E < 1 || f < 1 || d < 1 || r < 1) return 0;
  return moe_grouped_ffn_workspace_size(R, E, d, f, MOE_BF16) + lora_extra_bytes(R, E, d, f, r);
}

// Byte offsets inside the LoRA workspace of the backward's rank-r rows:
// u_dn, store(w u_dn) and u_gu, each [R, r] bf16 (after the tile starts of
// the rank-r projections and the transposed B factors).
struct LoraBwdLayout {
  size_t ts16, b_dn_t, b_gu_t, u_dn, uw_dn, u_gu;
};
static LoraBwdLayout lora_bwd_layout(int64_t R, int E, int d, int f, int r) {
  LoraBwdLayout L;
  size_t o = moe_grouped_ffn_workspace_size(R, E, d, f, MOE_BF16);
  L.ts16 = o;
  o += tile_start_bytes(E);
  L.b_dn_t = o;
  o += align_up(2 * (size_t)E * r * d, 256);
  L.b_gu_t = o;
  o += align_up(2 * (size_t)E * r * 2 * f, 256);
  L.u_dn = o;
  o += align_up(2 * (size_t)R * r, 256);
  L.uw_dn = o;
  o += align_up(2 * (size_t)R * r, 256);
  L.u_gu = o;
  return L;
}

extern "C" int moe_grouped_ffn_lora_bwd_saved(const void *ws, size_t ws_bytes, int64_t R, int E,
                                              int d, int f, int r, const void **u_dn,
                                              const void **uw_dn, const void **u_gu) {
  clear_error();
  MOE_REQUIRE(ws && u_dn && uw_dn && u_gu, MOE_ERR_INVALID_ARG,
              "moe_grouped_ffn_lora_bwd_saved: null pointer");
  MOE_REQUIRE(R >= 0 && E >= 1 && d > 0 && f > 0 && (r == 16 || r == 32 || r == 48 || r == 64),
              MOE_ERR_INVALID_ARG, "moe_grouped_ffn_lora_bwd_saved: bad sizes");
  const size_t need = moe_grouped_ffn_lora_workspace_size(R, E, d, f, r);
  MOE_REQUIRE(ws_bytes >= need, MOE_ERR_WORKSPACE,
              "moe_grouped_ffn_lora_bwd_saved: workspace %zu < %zu", ws_bytes, need);
  const LoraBwdLayout L = lora_bwd_layout(R, E, d, f, r);
  const char *w = (const char *)ws;
  *u_dn = w + L.u_dn;
  *uw_dn = w + L.uw_dn;
  *u_gu = w + L.u_gu;
  return MOE_OK;
}

template <int RK>
static int launch_lora_proj(const bf16_t *in, const bf16_t *F, const int32_t *offsets,
                            const int32_t *ts, int E, int64_t R, int K, float scale, const float *w,
                            bf16_t *out, bf16_t *out_w, const char *name, hipStream_t s) {
  const unsigned blocks = (unsigned)((R + 15) / 16 + E);   // bound on 16-row tiles
  MOE_LAUNCH(name, s,
             k_lora_proj<RK><<<blocks, 256, 0, s>>>(in, F, offsets, ts, E, K, scale, w, out, out_w));
  return check_launch(name);
}

static int lora_proj(int r, const bf16_t *in, const bf16_t *F, const int32_t *offsets,
                     const int32_t *ts, int E, int64_t R, int K, float scale, const float *w,
                     bf16_t *out, bf16_t *out_w, const char *name, hipStream_t s) {
  switch (r) {
    case 16: return launch_lora_proj<16>(in, F, offsets, ts, E, R, K, scale, w, out, out_w, name, s);
    case 32: return launch_lora_proj<32>(in, F, offsets, ts, E, R, K, scale, w, out, out_w, name, s);
    case 48: return launch_lora_proj<48>(in, F, offsets, ts, E, R, K, scale, w, out, out_w, name, s);
    default: return launch_lora_proj<64>(in, F, offsets, ts, E, R, K, scale, w, out, out_w, name, s);
  }
}

template <int RK, bool KR>
static int launch_lora_grad_t(const bf16_t *M, const bf16_t *Z, const int32_t *offsets, int E,
                              int K, float *out, const char *name, hipStream_t s) {
  const unsigned blocks = (unsigned)(E * ((K + 255) / 256));
  MOE_LAUNCH(name, s, (k_lora_grad<RK, KR><<<blocks, 256, 0, s>>>(M, Z, offsets, E, K, out)));
  return check_launch(name);
}

template <bool KR>
static int lora_grad(int r, const bf16_t *M, const bf16_t *Z, const int32_t *offsets, int E, int K,
                     float *out, const char *name, hipStream_t s) {
  switch (r) {
    case 16: return launch_lora_grad_t<16, KR>(M, Z, offsets, E, K, out, name, s);
    case 32: return launch_lora_grad_t<32, KR>(M, Z, offsets, E, K, out, name, s);
    case 48: return launch_lora_grad_t<48, KR>(M, Z, offsets, E, K, out, name, s);
    default: return launch_lora_grad_t<64, KR>(M, Z, offsets, E, K, out, name, s);
  }
}

extern "C" int moe_grouped_ffn_fwd_lora(const void *x_perm, const int32_t *offsets, int E,
                                        int64_t R, int d, int f, const void *w_gu,
                                        const void *w_down, const float *row_scale,
                                        const void *a_gu, const void *b_gu, const void *a_dn,
                                        const void *b_dn, int r, float scale, int dtype,
                                        void *z_gu, void *z_dn, void *gu, void *h, void *y_perm,
                                        void *ws, size_t ws_bytes, void *stream) {
  clear_error();
  int rc = check_ffn("moe_grouped_ffn_fwd_lora", E, R, d, f, dtype);
  if (rc) return rc;
  rc = check_lora("moe_grouped_ffn_fwd_lora", r, scale);
  if (rc) return rc;
  MOE_REQUIRE(dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "moe_grouped_ffn_fwd_lora: needs MOE_BF16");
  if (R == 0) return MOE_OK;
  MOE_REQUIRE(x_perm && offsets && w_gu && w_down && a_gu && b_gu && a_dn && b_dn && z_gu &&
                  z_dn && h && y_perm,
              MOE_ERR_INVALID_ARG, "moe_grouped_ffn_fwd_lora: null pointer");
  MOE_REQUIRE(aligned16(x_perm) && aligned16(w_gu) && aligned16(w_down) && aligned16(a_gu) &&
                  aligned16(b_gu) && aligned16(a_dn) && aligned16(b_dn) && aligned16(z_gu) &&
                  aligned16(z_dn) && aligned16(h) && aligned16(y_perm) && (!gu || aligned16(gu)),
              MOE_ERR_INVALID_ARG, "moe_grouped_ffn_fwd_lora: pointers must be 16-byte aligned");
  const size_t need = moe_grouped_ffn_lora_workspace_size(R, E, d, f, r);
  MOE_REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE,
              "moe_grouped_ffn_fwd_lora: workspace %zu < %zu", ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  int32_t *ts0 = (int32_t *)ws;
  int32_t *ts1 = (int32_t *)((char *)ws + tile_start_bytes(E));
  int32_t *ts16 = (int32_t *)((char *)ws + moe_grouped_ffn_workspace_size(R, E, d, f, MOE_BF16));
  GemmArgs a{};
  a.x_perm = (const bf16_t *)x_perm;
  a.w_gu = (const bf16_t *)w_gu;
  a.w_down = (const bf16_t *)w_down;
  a.h = (const bf16_t *)h;
  a.row_scale = row_scale;
  a.offsets = offsets;
  a.o_gu = (bf16_t *)gu;
  a.o_h = (bf16_t *)h;
  a.o_y = (bf16_t *)y_perm;
  a.lora_r = r;
  a.E = E;
  a.d = d;
  a.f = f;
  const int pt_gu = (f + FWD_BP / 2 - 1) / (FWD_BP / 2), pt_dn = (d + DN_BP - 1) / DN_BP;
  rc = launch_tile_prefix(a, FWD_BQ, pt_gu, ts0, DN_BQ, pt_dn, ts1, s);
  if (rc) return rc;
  rc = launch_tile_prefix(a, 16, 1, ts16, 16, 1, ts16, s);   // 16-row tiles of the projections
  if (rc) return rc;
  // z_gu = store(s X_perm A_gu^T); GU and H with the extra K stage z_gu . B_gu^T
  rc = lora_proj(r, (const bf16_t *)x_perm, (const bf16_t *)a_gu, offsets, ts16, E, R, d, scale,
                 nullptr, (bf16_t *)z_gu, nullptr, "lora_proj", s);
  if (rc) return rc;
  a.lora_p = (const bf16_t *)b_gu;
  a.lora_q = (const bf16_t *)z_gu;
  rc = launch_token_gemm<FWD_GU, FWD_BP, FWD_BQ, FWD_WP, FWD_WQ, FWD_NS, FWD_BK, true>(
      a, R, pt_gu, ts0, "gg_fwd_gate_up_swiglu", s);
  if (rc) return rc;
  // z_dn = store(s H A_dn^T); Y_perm with the extra K stage z_dn . B_dn^T
  rc = lora_proj(r, (const bf16_t *)h, (const bf16_t *)a_dn, offsets, ts16, E, R, f, scale,
                 nullptr, (bf16_t *)z_dn, nullptr, "lora_proj", s);
  if (rc) return rc;
  a.lora_p = (const bf16_t *)b_dn;
  a.lora_q = (const bf16_t *)z_dn;
  return launch_token_gemm<FWD_DOWN, DN_BP, DN_BQ, DN_WP, DN_WQ, DN_NS, DN_BK, true>(
      a, R, pt_dn, ts1, "gg_fwd_down_scale", s);
}

extern "C" int moe_grouped_ffn_bwd_lora(const void *x_perm, const void *gu, const void *h,
                                        const int32_t *offsets, int E, int64_t R, int d, int f,
                                        const void *w_gu, const void *w_down,
                                        const float *row_scale, const void *dy_perm,
                                        const void *a_gu, const void *b_gu, const void *a_dn,
                                        const void *b_dn, int r, float scale, const void *z_gu,
                                        const void *z_dn, int dtype, void *dgu, void *dx_perm,
                                        float *d_row_scale, float *da_gu, float *db_gu,
                                        float *da_dn, float *db_dn, void *ws, size_t ws_bytes,
                                        void *stream) {
  clear_error();
  int rc = check_ffn("moe_grouped_ffn_bwd_lora", E, R, d, f, dtype);
  if (rc) return rc;
  rc = check_lora("moe_grouped_ffn_bwd_lora", r, scale);
  if (rc) return rc;
  MOE_REQUIRE(dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "moe_grouped_ffn_bwd_lora: needs MOE_BF16");
  MOE_REQUIRE(offsets && w_gu && w_down && a_gu && b_gu && a_dn && b_dn && da_gu && db_gu &&
                  da_dn && db_dn,
              MOE_ERR_INVALID_ARG, "moe_grouped_ffn_bwd_lora: null pointer");
  MOE_REQUIRE(R == 0 || (x_perm && gu && h && dy_perm && z_gu && z_dn && dgu && dx_perm),
              MOE_ERR_INVALID_ARG, "moe_grouped_ffn_bwd_lora: null activation pointer");
  MOE_REQUIRE(aligned16(w_gu) && aligned16(w_down) && aligned16(a_gu) && aligned16(b_gu) &&
                  aligned16(a_dn) && aligned16(b_dn) &&
                  (R == 0 || (aligned16(x_perm) && aligned16(gu) && aligned16(h) &&
                              aligned16(dy_perm) && aligned16(z_gu) && aligned16(z_dn) &&
                              aligned16(dgu) && aligned16(dx_perm))),
              MOE_ERR_INVALID_ARG, "moe_grouped_ffn_bwd_lora: pointers must be 16-byte aligned");
  const size_t need = moe_grouped_ffn_lora_workspace_size(R, E, d, f, r);
  MOE_REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE,
              "moe_grouped_ffn_bwd_lora: workspace %zu < %zu", ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  char *wb = (char *)ws;
  int32_t *ts0 = (int32_t *)wb;
  int32_t *ts1 = (int32_t *)(wb + tile_start_bytes(E));
  float *drs_part = (float *)(wb + 2 * tile_start_bytes(E));
  bf16_t *s_perm = (bf16_t *)(wb + 2 * tile_start_bytes(E) + drs_bytes(R, f));
  const LoraBwdLayout L = lora_bwd_layout(R, E, d, f, r);
  int32_t *ts16 = (int32_t *)(wb + L.ts16);
  bf16_t *b_dn_t = (bf16_t *)(wb + L.b_dn_t);   // [E, r, d]
  bf16_t *b_gu_t = (bf16_t *)(wb + L.b_gu_t);   // [E, r, 2f]
  bf16_t *u_dn = (bf16_t *)(wb + L.u_dn);
  bf16_t *uw_dn = (bf16_t *)(wb + L.uw_dn);
  bf16_t *u_gu = (bf16_t *)(wb + L.u_gu);
  GemmArgs a{};
  a.x_perm = (const bf16_t *)x_perm;
  a.w_gu = (const bf16_t *)w_gu;
  a.w_down = (const bf16_t *)w_down;
  a.h = (const bf16_t *)h;
  a.gu = (const bf16_t *)gu;
  a.dy_perm = (const bf16_t *)dy_perm;
  a.dgu = (const bf16_t *)dgu;
  a.row_scale = row_scale;
  a.offsets = offsets;
  a.o_dgu = (bf16_t *)dgu;
  a.o_dx = (bf16_t *)dx_perm;
  a.o_drs = drs_part;
  a.lora_r = r;
  a.E = E;
  a.d = d;
  a.f = f;
  // B factors with K contiguous for the projections
  {
    MOE_LAUNCH("lora_transpose", s,
               k_lora_transpose<<<(unsigned)(E * ((d + 255) / 256)), 256, 0, s>>>(
                   (const bf16_t *)b_dn, E, d, r, b_dn_t));
    MOE_LAUNCH("lora_transpose", s,
               k_lora_transpose<<<(unsigned)(E * ((2 * f + 255) / 256)), 256, 0, s>>>(
                   (const bf16_t *)b_gu, E, 2 * f, r, b_gu_t));
    rc = check_launch("moe_grouped_ffn_bwd_lora(transpose)");
    if (rc) return rc;
  }
  const int pt_dh = (f + DH_BP - 1) / DH_BP, pt_dx = (d + DX_BP - 1) / DX_BP;
  if (R > 0) {
    rc = launch_tile_prefix(a, DH_BQ, pt_dh, ts0, DX_BQ, pt_dx, ts1, s);
    if (rc) return rc;
    rc = launch_tile_prefix(a, 16, 1, ts16, 16, 1, ts16, s);
    if (rc) return rc;
    // u_dn = store(s dY_perm B_dn), w * u_dn stored too
    rc = lora_proj(r, (const bf16_t *)dy_perm, b_dn_t, offsets, ts16, E, R, d, scale, row_scale
                   ? row_scale : nullptr, u_dn, row_scale ? uw_dn : nullptr, "lora_proj", s);
    if (rc) return rc;
    if (!row_scale) uw_dn = u_dn;
  }
  // 1. dGU (and d_row_scale partials): dY_perm W_down + u_dn A_dn
  a.lora_p = (const bf16_t *)a_dn;
  a.lora_q = u_dn;
  rc = launch_token_gemm<BWD_DH, DH_BP, DH_BQ, DH_WP, DH_WQ, DH_NS, DH_BK, true>(
      a, R, pt_dh, ts0, "gg_bwd_dh_dswiglu", s);
  if (rc) return rc;
  if (d_row_scale && R > 0) {
    MOE_LAUNCH("drs_reduce", s,
               k_drs_reduce<<<(unsigned)((R + 255) / 256), 256, 0, s>>>(drs_part, pt_dh * DH_WP, R,
                                                                       d_row_scale));
    rc = check_launch("moe_grouped_ffn_bwd_lora(drs)");
    if (rc) return rc;
  }
  // 2. u_gu = store(s dGU B_gu); dX_perm = dGU W_gu + u_gu A_gu
  if (R > 0) {
    rc = lora_proj(r, (const bf16_t *)dgu, b_gu_t, offsets, ts16, E, R, 2 * f, scale, nullptr,
                   u_gu, nullptr, "lora_proj", s);
    if (rc) return rc;
  }
  a.lora_p = (const bf16_t *)a_gu;
  a.lora_q = u_gu;
  rc = launch_token_gemm<BWD_DX, DX_BP, DX_BQ, DX_WP, DX_WQ, DX_NS, DX_BK, true>(
      a, R, pt_dx, ts1, "gg_bwd_dx", s);
  if (rc) return rc;
  // 3. S = store(w dY_perm) for dB_dn
  if (R > 0) {
    MOE_LAUNCH("row_scale", s,
               k_row_scale<<<(unsigned)((R + 3) / 4), 256, 0, s>>>(
                   (const bf16_t *)dy_perm, row_scale, R, d, s_perm));
    rc = check_launch("moe_grouped_ffn_bwd_lora(row scale)");
    if (rc) return rc;
  }
  // 4. factor gradients (fp32): dB_gu = dGU^T z_gu, dA_gu = u_gu^T X_perm,
  //    dB_dn = S^T z_dn, dA_dn = store(w u_dn)^T H
  rc = lora_grad<true>(r, (const bf16_t *)dgu, (const bf16_t *)z_gu, offsets, E, 2 * f, db_gu,
                       "lora_grad", s);
  if (rc) return rc;
  rc = lora_grad<false>(r, (const bf16_t *)x_perm, u_gu, offsets, E, d, da_gu, "lora_grad", s);
  if (rc) return rc;
  rc = lora_grad<true>(r, s_perm, (const bf16_t *)z_dn, offsets, E, d, db_dn, "lora_grad", s);
  if (rc) return rc;
  return lora_grad<false>(r, (const bf16_t *)h, uw_dn, offsets, E, f, da_dn, "lora_grad", s);
}
