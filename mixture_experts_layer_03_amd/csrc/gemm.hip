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
#include "moe_internal.h"

namespace moe {

enum GemmKind { FWD_GU = 0, FWD_DOWN = 1, BWD_DH = 2, BWD_DX = 3, BWD_DWDOWN = 4, BWD_DWGU = 5 };

constexpr int kBK = 64;   // k per LDS stage: 64 bf16 = 128 bytes = 8 chunks per row

struct GemmArgs {
  // operands
  const bf16_t *x_perm, *w_gu, *w_down, *h, *gu, *dy_perm, *dgu;
  const float *row_scale;      // [R] or null
  const int32_t *offsets;      // [E+1]
  const int32_t *tile_start;   // [E+1] (token-tiled kinds)
  // outputs
  bf16_t *o_gu, *o_h, *o_y, *o_dgu, *o_dx;
  float *o_dw, *o_drs;         // dw: [E, Qdim, Pdim]; drs partials [R, PT*WP]
  int E, d, f;
  int PT;                      // tiles along P
  int QT;                      // tiles along Q (weight-gradient kinds)
  int nlogical;                // weight-gradient kinds: E*PT*QT
};

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ u32x4_t ld16(const bf16_t *p) {
  return *reinterpret_cast<const u32x4_t *>(p);
}

// chunk slot of (row, chunk) in a [rows][8 chunks] LDS tile, xor-swizzled so
// that 8 consecutive rows reading the same chunk hit 8 different bank groups
__device__ __forceinline__ int swz(int row, int ch) { return row * 8 + (ch ^ (row & 7)); }

// 8x8 transpose of bf16: in[i] = 8 values of k-row i (cols 0..7);
// out[c] = 8 values of column c (k rows 0..7).
__device__ __forceinline__ void transpose8x8(const u32x4_t in[8], u32x4_t out[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t a = in[2 * m][w], b = in[2 * m + 1][w];
      out[c][m] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
}

// scale the 8 bf16 of v by s and round back to bf16
__device__ __forceinline__ u32x4_t scale_bf16x8(u32x4_t v, float s) {
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = bf16_bits_to_f32(v[i] & 0xffffu) * s;
    const float hi = bf16_bits_to_f32(v[i] >> 16) * s;
    o[i] = pack_bf16x2(lo, hi);
  }
  return o;
}

// ------------------------------------------------------------------ loaders
//
// KContig operand tile: ROWS rows x 64 k, element (i,k) at base[i*ld + k]
// (paired: rows >= ROWS/2 come from base2).  Unit u = (row u/8, chunk u%8).
template <int ROWS, int NTHR>
struct KContigLoader {
  static constexpr int UNITS = ROWS * 8;
  static constexpr int NU = (UNITS + NTHR - 1) / NTHR;
  u32x4_t v[NU];

  __device__ __forceinline__ void load(const bf16_t *base, const bf16_t *base2, int64_t ld,
                                       int rows_valid, int k0, int kvalid, int tid) {
#pragma unroll
    for (int n = 0; n < NU; ++n) {
      const int u = tid + n * NTHR;
      v[n] = u32x4_t{0, 0, 0, 0};
      if (UNITS % NTHR == 0 || u < UNITS) {
        int row = u >> 3;
        const int k = k0 + (u & 7) * 8;
        const bf16_t *b = base;
        if (base2 && row >= ROWS / 2) {
          b = base2;
          row -= ROWS / 2;
        }
        if (row < rows_valid && k < kvalid) v[n] = ld16(b + (int64_t)row * ld + k);
      }
    }
  }
  __device__ __forceinline__ void store(u32x4_t *lds, int tid) const {
#pragma unroll
    for (int n = 0; n < NU; ++n) {
      const int u = tid + n * NTHR;
      if (UNITS % NTHR == 0 || u < UNITS) lds[swz(u >> 3, u & 7)] = v[n];
    }
  }
};

// Transposed operand tile: ROWS output rows x 64 k, element (i,k) at
// base[k*ld + i].  Unit u = (k block u%8, row block u/8); optional per-k
// scale (the row weight of the down-projection weight gradient).
template <int ROWS, int NTHR>
struct TransLoader {
  static constexpr int UNITS = ROWS;   // (ROWS/8) row blocks x 8 k blocks
  static constexpr int NU = (UNITS + NTHR - 1) / NTHR;
  u32x4_t v[NU][8];

  __device__ __forceinline__ void load(const bf16_t *base, int64_t ld, int rows_valid, int k0,
                                       int kvalid, const float *kscale, int tid) {
#pragma unroll
    for (int n = 0; n < NU; ++n) {
      const int u = tid + n * NTHR;
      const bool live = (UNITS % NTHR == 0) || u < UNITS;
      const int kb = u & 7, rb = u >> 3;
      const bool colok = live && rb * 8 < rows_valid;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = k0 + kb * 8 + i;
        v[n][i] = u32x4_t{0, 0, 0, 0};
        if (colok && k < kvalid) {
          v[n][i] = ld16(base + (int64_t)k * ld + rb * 8);
          if (kscale) v[n][i] = scale_bf16x8(v[n][i], kscale[k]);
        }
      }
    }
  }
  __device__ __forceinline__ void store(u32x4_t *lds, int tid) const {
#pragma unroll
    for (int n = 0; n < NU; ++n) {
      const int u = tid + n * NTHR;
      if ((UNITS % NTHR == 0) || u < UNITS) {
        const int kb = u & 7, rb = u >> 3;
        u32x4_t t[8];
        transpose8x8(v[n], t);
#pragma unroll
        for (int c = 0; c < 8; ++c) lds[swz(rb * 8 + c, kb)] = t[c];
      }
    }
  }
};

template <int KIND> struct KindTraits;
template <> struct KindTraits<FWD_GU>     { static constexpr bool PT_ = false, QT_ = false, PAIRED = true,  WG = false; };
template <> struct KindTraits<FWD_DOWN>   { static constexpr bool PT_ = false, QT_ = false, PAIRED = false, WG = false; };
template <> struct KindTraits<BWD_DH>     { static constexpr bool PT_ = true,  QT_ = false, PAIRED = false, WG = false; };
template <> struct KindTraits<BWD_DX>     { static constexpr bool PT_ = true,  QT_ = false, PAIRED = false, WG = false; };
template <> struct KindTraits<BWD_DWDOWN> { static constexpr bool PT_ = true,  QT_ = true,  PAIRED = false, WG = true; };
template <> struct KindTraits<BWD_DWGU>   { static constexpr bool PT_ = true,  QT_ = true,  PAIRED = false, WG = true; };

template <bool TRANS, int ROWS, int NTHR> struct LoaderSel;
template <int ROWS, int NTHR> struct LoaderSel<false, ROWS, NTHR> { typedef KContigLoader<ROWS, NTHR> type; };
template <int ROWS, int NTHR> struct LoaderSel<true, ROWS, NTHR>  { typedef TransLoader<ROWS, NTHR> type; };

// Operand description for one tile.
struct Opnd {
  const bf16_t *base;
  const bf16_t *base2;   // paired second half (KContig only)
  int64_t ld;
  int rows_valid;
  int kvalid;
  const float *kscale;   // transposed only
};

template <typename L>
__device__ __forceinline__ void load_op(L &l, const Opnd &o, int k0, int tid);
template <int R, int N>
__device__ __forceinline__ void load_op(KContigLoader<R, N> &l, const Opnd &o, int k0, int tid) {
  l.load(o.base, o.base2, o.ld, o.rows_valid, k0, o.kvalid, tid);
}
template <int R, int N>
__device__ __forceinline__ void load_op(TransLoader<R, N> &l, const Opnd &o, int k0, int tid) {
  l.load(o.base + (int64_t)k0 * o.ld, o.ld, o.rows_valid, 0, o.kvalid - k0, o.kscale ? o.kscale + k0 : nullptr, tid);
}

// ------------------------------------------------------------------ kernel

template <int KIND, int BP, int BQ, int WP, int WQ>
__global__ __launch_bounds__(WP *WQ * 64) void k_grouped_gemm(GemmArgs a) {
  using KT = KindTraits<KIND>;
  constexpr int NTHR = WP * WQ * 64;
  constexpr int FP = BP / WP / 16;
  constexpr int FQ = BQ / WQ / 16;
  static_assert(FP >= 1 && FQ >= 1, "tile too small");
  static_assert(!KT::PAIRED || (FP % 2 == 0), "paired tiles need an even fragment count");
  using PL = typename LoaderSel<KT::PT_, BP, NTHR>::type;
  using QL = typename LoaderSel<KT::QT_, BQ, NTHR>::type;

  __shared__ u32x4_t lds[2][(BP + BQ) * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wp = wave % WP, wq = wave / WP;
  const int qtid = tid ^ (NTHR / 2);   // spread the Q loader over the other half first

  // ---- XCD-aware tile order: workgroups are dealt round-robin over the 8
  // XCDs; give each XCD a contiguous range of logical tiles.
  const int nb = gridDim.x;
  const int b = blockIdx.x;
  const int L = (b & 7) * (nb >> 3) + (b >> 3);

  int e, p_tile, q_tile, seg0, Me;
  if (KT::WG) {
    if (L >= a.nlogical) return;
    const int per_e = a.PT * a.QT;
    e = L / per_e;
    const int rem = L - e * per_e;
    p_tile = rem / a.QT;
    q_tile = rem - p_tile * a.QT;
    seg0 = a.offsets[e];
    Me = a.offsets[e + 1] - seg0;
  } else {
    const int total = a.tile_start[a.E];
    if (L >= total) return;
    int lo = 0, hi = a.E;   // largest e with tile_start[e] <= L
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.tile_start[mid] <= L) lo = mid; else hi = mid;
    }
    e = lo;
    seg0 = a.offsets[e];
    Me = a.offsets[e + 1] - seg0;
    const int qt_e = (Me + BQ - 1) / BQ;
    const int rem = L - a.tile_start[e];
    p_tile = rem / qt_e;
    q_tile = rem - p_tile * qt_e;
  }
  const int d = a.d, f = a.f;
  const int64_t f2 = 2 * (int64_t)f;

  // ---- operands of this tile
  Opnd P{}, Q{};
  int K = 0;
  const int p0 = p_tile * (KT::PAIRED ? BP / 2 : BP);
  const int q0 = q_tile * BQ;
  if (KIND == FWD_GU) {
    const bf16_t *W = a.w_gu + (int64_t)e * f2 * d;
    P = Opnd{W + (int64_t)p0 * d, W + ((int64_t)f + p0) * d, d, f - p0, d, nullptr};
    Q = Opnd{a.x_perm + ((int64_t)seg0 + q0) * d, nullptr, d, Me - q0, d, nullptr};
    K = d;
  } else if (KIND == FWD_DOWN) {
    const bf16_t *W = a.w_down + (int64_t)e * d * f;
    P = Opnd{W + (int64_t)p0 * f, nullptr, f, d - p0, f, nullptr};
    Q = Opnd{a.h + ((int64_t)seg0 + q0) * f, nullptr, f, Me - q0, f, nullptr};
    K = f;
  } else if (KIND == BWD_DH) {
    const bf16_t *W = a.w_down + (int64_t)e * d * f;
    P = Opnd{W + p0, nullptr, f, f - p0, d, nullptr};
    Q = Opnd{a.dy_perm + ((int64_t)seg0 + q0) * d, nullptr, d, Me - q0, d, nullptr};
    K = d;
  } else if (KIND == BWD_DX) {
    const bf16_t *W = a.w_gu + (int64_t)e * f2 * d;
    P = Opnd{W + p0, nullptr, d, d - p0, (int)f2, nullptr};
    Q = Opnd{a.dgu + ((int64_t)seg0 + q0) * f2, nullptr, f2, Me - q0, (int)f2, nullptr};
    K = (int)f2;
  } else if (KIND == BWD_DWDOWN) {
    P = Opnd{a.h + (int64_t)seg0 * f + p0, nullptr, f, f - p0, Me, nullptr};
    Q = Opnd{a.dy_perm + (int64_t)seg0 * d + q0, nullptr, d, d - q0, Me,
             a.row_scale ? a.row_scale + seg0 : nullptr};
    K = Me;
  } else {   // BWD_DWGU
    P = Opnd{a.x_perm + (int64_t)seg0 * d + p0, nullptr, d, d - p0, Me, nullptr};
    Q = Opnd{a.dgu + (int64_t)seg0 * f2 + q0, nullptr, f2, (int)(f2 - q0), Me, nullptr};
    K = Me;
  }

  f32x4_t acc[FP][FQ];
#pragma unroll
  for (int i = 0; i < FP; ++i)
#pragma unroll
    for (int j = 0; j < FQ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // fragment rows inside the LDS tiles
  int prow[FP], qrow[FQ];
#pragma unroll
  for (int i = 0; i < FP; ++i) {
    if (KT::PAIRED) {
      constexpr int HALF = BP / 2, PW = BP / 2 / WP;
      prow[i] = (i < FP / 2) ? wp * PW + i * 16 : HALF + wp * PW + (i - FP / 2) * 16;
    } else {
      prow[i] = wp * (BP / WP) + i * 16;
    }
  }
#pragma unroll
  for (int j = 0; j < FQ; ++j) qrow[j] = wq * (BQ / WQ) + j * 16;

  const int nk = (K + kBK - 1) / kBK;
  if (nk > 0) {
    PL pl;
    QL ql;
    load_op(pl, P, 0, tid);
    load_op(ql, Q, 0, qtid);
    pl.store(&lds[0][0], tid);
    ql.store(&lds[0][BP * 8], qtid);
    __syncthreads();
    const int fr = lane & 15, fg = lane >> 4;
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) {
        load_op(pl, P, (kt + 1) * kBK, tid);
        load_op(ql, Q, (kt + 1) * kBK, qtid);
      }
      const u32x4_t *lp = &lds[cur][0];
      const u32x4_t *lq = &lds[cur][BP * 8];
#pragma unroll
      for (int ks = 0; ks < kBK / 32; ++ks) {
        bf16x8_t pf[FP], qf[FQ];
#pragma unroll
        for (int i = 0; i < FP; ++i) pf[i] = as_bf16x8(lp[swz(prow[i] + fr, ks * 4 + fg)]);
#pragma unroll
        for (int j = 0; j < FQ; ++j) qf[j] = as_bf16x8(lq[swz(qrow[j] + fr, ks * 4 + fg)]);
#pragma unroll
        for (int i = 0; i < FP; ++i)
#pragma unroll
          for (int j = 0; j < FQ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[i], qf[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) {
        pl.store(&lds[cur ^ 1][0], tid);
        ql.store(&lds[cur ^ 1][BP * 8], qtid);
      }
      __syncthreads();
    }
  }

  // ---- epilogues.  Lane holds D[prow+4*(lane/16)+v][qrow+lane%16].
  const int er = 4 * (lane >> 4);
  const int ec = lane & 15;
  if (KIND == FWD_GU) {
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
          hv[v] = g[v] / (1.0f + __expf(-g[v])) * u[v];
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
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      const int q = q0 + qrow[j] + ec;
      if (q >= Me) continue;
      const int64_t r = (int64_t)seg0 + q;
      const float w = (KIND == FWD_DOWN && a.row_scale) ? a.row_scale[r] : 1.0f;
#pragma unroll
      for (int i = 0; i < FP; ++i) {
        const int n = p0 + prow[i] + er;
        if (n >= d) continue;
        *reinterpret_cast<u32x2_t *>(out + r * d + n) =
            u32x2_t{pack_bf16x2(w * acc[i][j][0], w * acc[i][j][1]),
                    pack_bf16x2(w * acc[i][j][2], w * acc[i][j][3])};
      }
    }
  } else if (KIND == BWD_DH) {
    const int nparts = a.PT * WP;
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      const int q = q0 + qrow[j] + ec;
      const bool rowok = q < Me;
      const int64_t r = (int64_t)seg0 + (rowok ? q : 0);
      const float w = (rowok && a.row_scale) ? a.row_scale[r] : 1.0f;
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < FP; ++i) {
        const int c = p0 + prow[i] + er;
        if (!rowok || c >= f) continue;
        const u32x2_t g2 = *reinterpret_cast<const u32x2_t *>(a.gu + r * f2 + c);
        const u32x2_t u2 = *reinterpret_cast<const u32x2_t *>(a.gu + r * f2 + f + c);
        const u32x2_t h2 = *reinterpret_cast<const u32x2_t *>(a.h + r * f + c);
        float dg[4], du[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t gw = g2[v >> 1], uw = u2[v >> 1], hw = h2[v >> 1];
          const float g = bf16_bits_to_f32((v & 1) ? (gw >> 16) : (gw & 0xffffu));
          const float u = bf16_bits_to_f32((v & 1) ? (uw >> 16) : (uw & 0xffffu));
          const float hv = bf16_bits_to_f32((v & 1) ? (hw >> 16) : (hw & 0xffffu));
          const float sg = 1.0f / (1.0f + __expf(-g));
          const float silu = g * sg;
          const float gd = acc[i][j][v];
          part += hv * gd;
          const float dh = w * gd;
          dg[v] = dh * u * sg * (1.0f + g * (1.0f - sg));
          du[v] = dh * silu;
        }
        *reinterpret_cast<u32x2_t *>(a.o_dgu + r * f2 + c) =
            u32x2_t{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
        *reinterpret_cast<u32x2_t *>(a.o_dgu + r * f2 + f + c) =
            u32x2_t{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
      }
      // sum over the 4 lane groups that share this token (fixed order)
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      if (a.o_drs && rowok && lane < 16)
        a.o_drs[r * nparts + p_tile * WP + wp] = part;
    }
  } else {   // weight gradients: dw[e][q][p]
    const int Pdim = (KIND == BWD_DWDOWN) ? f : d;
    const int Qdim = (KIND == BWD_DWDOWN) ? d : (int)f2;
    float *out = a.o_dw + (int64_t)e * Pdim * Qdim;
#pragma unroll
    for (int j = 0; j < FQ; ++j) {
      const int q = q0 + qrow[j] + ec;
      if (q >= Qdim) continue;
#pragma unroll
      for (int i = 0; i < FP; ++i) {
        const int p = p0 + prow[i] + er;
        if (p >= Pdim) continue;
        *reinterpret_cast<f32x4_t *>(out + (int64_t)q * Pdim + p) = acc[i][j];
      }
    }
  }
}

// tile_start[e] = sum over e' < e of ceil(M_e' / BQ) * PT  (one block)
__global__ __launch_bounds__(1024) void k_tile_prefix(const int32_t *__restrict__ offsets, int E,
                                                      int BQ, int PT,
                                                      int32_t *__restrict__ tile_start) {
  __shared__ int s[1024];
  const int e = threadIdx.x;
  int v = 0;
  if (e < E) {
    const int m = offsets[e + 1] - offsets[e];
    v = (m + BQ - 1) / BQ * PT;
  }
  s[e] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int t = e >= off ? s[e - off] : 0;
    __syncthreads();
    s[e] += t;
    __syncthreads();
  }
  if (e < E) tile_start[e + 1] = s[e];
  if (e == 0) tile_start[0] = 0;
}

// d_row_scale[r] = sum of its partials in fixed order
__global__ __launch_bounds__(256) void k_drs_reduce(const float *__restrict__ part, int nparts,
                                                    int64_t R, float *__restrict__ drs) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  float s = 0.0f;
  for (int i = 0; i < nparts; ++i) s += part[r * nparts + i];
  drs[r] = s;
}

// ------------------------------------------------------------------ fp32 forward
//
// fp32 storage (no MFMA bf16 path): one thread per (row, 4 features), fp32
// fma over k in order.  Used for fp32 workloads only.
__global__ __launch_bounds__(256) void k_ffn_gu_f32(const float *__restrict__ x_perm,
                                                    const int32_t *__restrict__ offsets, int E,
                                                    int64_t R, int d, int f,
                                                    const float *__restrict__ w_gu,
                                                    float *__restrict__ gu, float *__restrict__ h) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nq = f / 4;
  if (i >= R * nq) return;
  const int64_t r = i / nq;
  const int n = (int)(i % nq) * 4;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  const int e = lo;
  if (r < offsets[e] || r >= offsets[e + 1]) return;
  const float *x = x_perm + r * d;
  const float *wg = w_gu + ((int64_t)e * 2 * f + n) * d;
  const float *wu = w_gu + ((int64_t)e * 2 * f + f + n) * d;
  float g[4] = {0, 0, 0, 0}, u[4] = {0, 0, 0, 0};
  for (int c = 0; c < d; ++c) {
    const float xv = x[c];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      g[v] = fmaf(xv, wg[(int64_t)v * d + c], g[v]);
      u[v] = fmaf(xv, wu[(int64_t)v * d + c], u[v]);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    if (gu) {
      gu[r * 2 * f + n + v] = g[v];
      gu[r * 2 * f + f + n + v] = u[v];
    }
    h[r * f + n + v] = g[v] / (1.0f + expf(-g[v])) * u[v];
  }
}

__global__ __launch_bounds__(256) void k_ffn_down_f32(const float *__restrict__ h,
                                                      const int32_t *__restrict__ offsets, int E,
                                                      int64_t R, int d, int f,
                                                      const float *__restrict__ w_down,
                                                      const float *__restrict__ row_scale,
                                                      float *__restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nq = d / 4;
  if (i >= R * nq) return;
  const int64_t r = i / nq;
  const int n = (int)(i % nq) * 4;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  const int e = lo;
  if (r < offsets[e] || r >= offsets[e + 1]) return;
  const float *hr = h + r * f;
  const float *wd = w_down + ((int64_t)e * d + n) * f;
  float acc[4] = {0, 0, 0, 0};
  for (int c = 0; c < f; ++c) {
    const float hv = hr[c];
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = fmaf(hv, wd[(int64_t)v * f + c], acc[v]);
  }
  const float w = row_scale ? row_scale[r] : 1.0f;
#pragma unroll
  for (int v = 0; v < 4; ++v) y[r * d + n + v] = w * acc[v];
}

// ------------------------------------------------------------------ launch

// tile configurations
constexpr int FWD_BP = 256, FWD_BQ = 128, FWD_WP = 2, FWD_WQ = 2;   // FWD_GU (P = gate|up pairs)
constexpr int DN_BP = 256, DN_BQ = 128, DN_WP = 2, DN_WQ = 2;       // FWD_DOWN, BWD_DX
constexpr int DH_BP = 128, DH_BQ = 128, DH_WP = 2, DH_WQ = 2;       // BWD_DH
constexpr int WG_BP = 128, WG_BQ = 128, WG_WP = 2, WG_WQ = 2;       // weight gradients

static inline int pad8(int64_t n) { return (int)((n + 7) / 8 * 8); }

template <int KIND, int BP, int BQ, int WP, int WQ>
static int launch_token_gemm(GemmArgs a, int64_t R, int PT, int32_t *tile_start, const char *name,
                             hipStream_t s) {
  if (R == 0) return MOE_OK;
  a.PT = PT;
  a.tile_start = tile_start;
  MOE_LAUNCH("tile_prefix", s,
             k_tile_prefix<<<1, 1024, 0, s>>>(a.offsets, a.E, BQ, PT, tile_start));
  const int64_t bound = ((R + BQ - 1) / BQ + a.E) * (int64_t)PT;
  const int grid = pad8(bound);
  MOE_LAUNCH(name, s, (k_grouped_gemm<KIND, BP, BQ, WP, WQ><<<grid, WP * WQ * 64, 0, s>>>(a)));
  return check_launch(name);
}

template <int KIND, int BP, int BQ, int WP, int WQ>
static int launch_wgrad_gemm(GemmArgs a, int Pdim, int Qdim, const char *name, hipStream_t s) {
  a.PT = (Pdim + BP - 1) / BP;
  a.QT = (Qdim + BQ - 1) / BQ;
  a.nlogical = a.E * a.PT * a.QT;
  const int grid = pad8(a.nlogical);
  MOE_LAUNCH(name, s, (k_grouped_gemm<KIND, BP, BQ, WP, WQ><<<grid, WP * WQ * 64, 0, s>>>(a)));
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

static size_t tile_start_bytes(int E) { return align_up(sizeof(int32_t) * (size_t)(E + 1), 256); }

extern "C" size_t moe_grouped_ffn_workspace_size(int64_t R, int E, int d, int f, int dtype) {
  (void)d;
  (void)dtype;
  if (R < 0 || E < 1 || f < 1) return 0;
  const int nparts = (f + DH_BP - 1) / DH_BP * DH_WP;
  return 2 * tile_start_bytes(E) + align_up(sizeof(float) * (size_t)R * nparts, 256);
}

extern "C" int moe_grouped_ffn_fwd(const void *x_perm, const int32_t *offsets, int E, int64_t R,
                                   int d, int f, const void *w_gu, const void *w_down,
                                   const float *row_scale, int dtype, void *gu, void *h,
                                   void *y_perm, void *ws, size_t ws_bytes, void *stream) {
  clear_error();
  int rc = check_ffn("moe_grouped_ffn_fwd", E, R, d, f, dtype);
  if (rc) return rc;
  if (R == 0) return MOE_OK;
  MOE_REQUIRE(x_perm && offsets && w_gu && w_down && h && y_perm, MOE_ERR_INVALID_ARG,
              "moe_grouped_ffn_fwd: null pointer");
  MOE_REQUIRE(aligned16(x_perm) && aligned16(w_gu) && aligned16(w_down) && aligned16(h) &&
                  aligned16(y_perm) && (!gu || aligned16(gu)),
              MOE_ERR_INVALID_ARG, "moe_grouped_ffn_fwd: pointers must be 16-byte aligned");
  const size_t need = moe_grouped_ffn_workspace_size(R, E, d, f, dtype);
  MOE_REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE, "moe_grouped_ffn_fwd: workspace %zu < %zu",
              ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == MOE_F32) {
    const int64_t n1 = R * (f / 4), n2 = R * (d / 4);
    MOE_LAUNCH("ffn_gu_f32", s,
               k_ffn_gu_f32<<<(unsigned)((n1 + 255) / 256), 256, 0, s>>>(
                   (const float *)x_perm, offsets, E, R, d, f, (const float *)w_gu, (float *)gu,
                   (float *)h));
    rc = check_launch("moe_grouped_ffn_fwd(gu f32)");
    if (rc) return rc;
    MOE_LAUNCH("ffn_down_f32", s,
               k_ffn_down_f32<<<(unsigned)((n2 + 255) / 256), 256, 0, s>>>(
                   (const float *)h, offsets, E, R, d, f, (const float *)w_down, row_scale,
                   (float *)y_perm));
    return check_launch("moe_grouped_ffn_fwd(down f32)");
  }
  int32_t *ts0 = (int32_t *)ws;
  int32_t *ts1 = (int32_t *)((char *)ws + tile_start_bytes(E));
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
  rc = launch_token_gemm<FWD_GU, FWD_BP, FWD_BQ, FWD_WP, FWD_WQ>(
      a, R, (f + FWD_BP / 2 - 1) / (FWD_BP / 2), ts0, "gg_fwd_gate_up_swiglu", s);
  if (rc) return rc;
  return launch_token_gemm<FWD_DOWN, DN_BP, DN_BQ, DN_WP, DN_WQ>(
      a, R, (d + DN_BP - 1) / DN_BP, ts1, "gg_fwd_down_scale", s);
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
  int32_t *ts0 = (int32_t *)ws;
  int32_t *ts1 = (int32_t *)((char *)ws + tile_start_bytes(E));
  float *drs_part = (float *)((char *)ws + 2 * tile_start_bytes(E));
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
  a.E = E;
  a.d = d;
  a.f = f;
  const int pt_dh = (f + DH_BP - 1) / DH_BP;
  // 1. dGU (and d_row_scale partials) from dY_perm and W_down
  rc = launch_token_gemm<BWD_DH, DH_BP, DH_BQ, DH_WP, DH_WQ>(a, R, pt_dh, ts0,
                                                             "gg_bwd_dh_dswiglu", s);
  if (rc) return rc;
  if (d_row_scale && R > 0) {
    MOE_LAUNCH("drs_reduce", s,
               k_drs_reduce<<<(unsigned)((R + 255) / 256), 256, 0, s>>>(drs_part, pt_dh * DH_WP, R,
                                                                       d_row_scale));
    rc = check_launch("moe_grouped_ffn_bwd(drs)");
    if (rc) return rc;
  }
  // 2. dX_perm = dGU . W_gu
  rc = launch_token_gemm<BWD_DX, DN_BP, DN_BQ, DN_WP, DN_WQ>(a, R, (d + DN_BP - 1) / DN_BP, ts1,
                                                             "gg_bwd_dx", s);
  if (rc) return rc;
  // 3. dW_down[e] = (w*dY_perm)^T H   -> [E, d, f]
  a.o_dw = dw_down;
  rc = launch_wgrad_gemm<BWD_DWDOWN, WG_BP, WG_BQ, WG_WP, WG_WQ>(a, f, d, "gg_bwd_dw_down", s);
  if (rc) return rc;
  // 4. dW_gu[e] = dGU^T X_perm        -> [E, 2f, d]
  a.o_dw = dw_gu;
  return launch_wgrad_gemm<BWD_DWGU, WG_BP, WG_BQ, WG_WP, WG_WQ>(a, d, 2 * f, "gg_bwd_dw_gate_up",
                                                                s);
}
