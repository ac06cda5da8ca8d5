// Router: fp32 logits, wavefront top-k + softmax over the selected k, and
// their adjoints.
//
// The pages: the EP forward path starts from "fp32 router logits" and a
// per-token top-k router whose probabilities weight the returned rows ("Halo's
// 2.8x over TRL is not a kernel, and its own benchmark proves it", section
// "Where the gap actually is").  Routers are trained, so they get gradients.
#include "moe_internal.h"

namespace moe {

// ------------------------------------------------------------------ logits
//
// Each (t,e) output is ONE fp32 fma chain over c = 0..d-1 in order, then
// + bias, then + noise, so the work per output cannot be split; there are
// T*E chains of d dependent fmas.  Block: 256 threads = 8 tokens x 32
// experts; wave w covers the block's 8 tokens x experts 8w..8w+7, lane l
// token l/8 and expert l%8, one chain per lane (T=4096, E=32 gives two waves
// per SIMD).  With many chains (T*E >= 2^20) a lane runs 4 tokens x 1 expert
// or 2 x 2 and the block covers 4 (2) times the tokens (and 2 times the
// experts): each LDS read then feeds several chains (the kernel reads both
// operands from LDS for every fma: LDS reads and instruction issue bound it).  Operands
// come from LDS tiles of logit_cols<TB>() columns (fp32, rows padded so that
// the 8 distinct rows one read touches fall on distinct banks; the 8 lanes
// that share a row read it as a broadcast); the next tile's global loads are
// in flight while the current one is used (widened to fp32 only when
// staged).  One chain per lane (few chains, two waves per SIMD) takes tiles
// of 256 columns, as wide as one 16-byte x load per thread allows, so that a
// tile's fmas cover more of the next tile's load latency: 38.6-39.3 -> 34.5-35.5
// us at T = 4096, E = 32.  The blocked forms keep 64 (at 128 the 2 x 2 form
// at T = 32768, E = 128 ran 366-369 -> 383-386 us: its larger LDS tiles
// leave fewer blocks per CU).
constexpr int kLogitTok = 8;     // tokens per block
constexpr int kLogitExp = 32;    // experts per block
template <int TB>
constexpr int logit_cols() { return TB == 1 ? 256 : 64; }   // columns per LDS tile

// 8 consecutive elements, raw
struct Raw8 {
  u32x4_t a, b;
};
__device__ __forceinline__ void load8_raw(const bf16_t *p, Raw8 &r) {
  r.a = *reinterpret_cast<const u32x4_t *>(p);
}
__device__ __forceinline__ void load8_raw(const float *p, Raw8 &r) {
  r.a = *reinterpret_cast<const u32x4_t *>(p);
  r.b = *reinterpret_cast<const u32x4_t *>(p + 4);
}
template <typename T>
__device__ __forceinline__ void widen8(const Raw8 &r, float *f) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_bits_to_f32(r.a[i] & 0xffffu);
      f[2 * i + 1] = bf16_bits_to_f32(r.a[i] >> 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = __uint_as_float(r.a[i]);
      f[4 + i] = __uint_as_float(r.b[i]);
    }
  }
}

// TB x EB chains per lane (tokens tok + 8i, experts el + 32j): a block covers
// 8*TB tokens x 32*EB experts, and every operand read from LDS feeds EB (or
// TB) chains.  Each chain keeps its own order.  Many chains (large T*E) use
// the blocked forms; few chains need every lane busy with one.
template <typename T, int TB, int EB>
__global__ __launch_bounds__(256) void k_router_logits(const T *__restrict__ x,
                                                       const T *__restrict__ wr,
                                                       const float *__restrict__ bias,
                                                       const float *__restrict__ noise,
                                                       int64_t ntok, int d, int E,
                                                       float *__restrict__ logits) {
  constexpr int NT = kLogitTok * TB, NE = kLogitExp * EB;   // block tokens, experts
  constexpr int CK = logit_cols<TB>(), PAD = CK + 4;         // tile columns, row pitch
  constexpr int UPR = CK / 8;                                 // 8-element units per tile row
  constexpr int XU = NT * UPR, WU = NE * UPR;                 // units of the x and w tiles
  static_assert(XU <= 256 && WU % 256 == 0, "at most one x unit, whole w units per thread");
  constexpr int WPT = WU / 256;
  __shared__ __attribute__((aligned(16))) float xs[NT][PAD];
  __shared__ __attribute__((aligned(16))) float ws[NE][PAD];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int tok = lane >> 3, el = wave * 8 + (lane & 7);
  const int64_t t0 = (int64_t)blockIdx.x * NT;
  const int e0 = blockIdx.y * NE;
  float acc[TB][EB];
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < EB; ++j) acc[i][j] = 0.0f;

  Raw8 xr, wrg[WPT];
  auto fetch = [&](int c0) {
    xr.a = xr.b = u32x4_t{0u, 0u, 0u, 0u};
    const int row = tid / UPR, col8 = (tid % UPR) * 8;
    if (tid < XU && t0 + row < ntok && c0 + col8 < d) load8_raw(x + (t0 + row) * d + c0 + col8, xr);
#pragma unroll
    for (int u = 0; u < WPT; ++u) {
      const int wu = tid + 256 * u, wrow = wu / UPR, wcol = (wu % UPR) * 8;
      wrg[u].a = wrg[u].b = u32x4_t{0u, 0u, 0u, 0u};
      if (e0 + wrow < E && c0 + wcol < d) load8_raw(wr + (int64_t)(e0 + wrow) * d + c0 + wcol, wrg[u]);
    }
  };
  auto stage = [&]() {
    float f[8];
    if (tid < XU) {
      const int row = tid / UPR, col8 = (tid % UPR) * 8;
      widen8<T>(xr, f);
      float *dst = &xs[row][col8];
      *reinterpret_cast<float4 *>(dst) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4 *>(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
    }
#pragma unroll
    for (int u = 0; u < WPT; ++u) {
      const int wu = tid + 256 * u, wrow = wu / UPR, wcol = (wu % UPR) * 8;
      widen8<T>(wrg[u], f);
      float *dst = &ws[wrow][wcol];
      *reinterpret_cast<float4 *>(dst) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4 *>(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
    }
  };

  fetch(0);
  for (int c0 = 0; c0 < d; c0 += CK) {
    stage();
    __syncthreads();
    if (c0 + CK < d) fetch(c0 + CK);
    const int cn = min(CK, d - c0);   // a multiple of 8
    auto step = [&](int cc) {
      float4 xv[TB], wv[EB];
#pragma unroll
      for (int i = 0; i < TB; ++i) xv[i] = *reinterpret_cast<const float4 *>(&xs[tok + 8 * i][cc]);
#pragma unroll
      for (int j = 0; j < EB; ++j) wv[j] = *reinterpret_cast<const float4 *>(&ws[el + 32 * j][cc]);
#pragma unroll
      for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int j = 0; j < EB; ++j) {
          acc[i][j] = fmaf(xv[i].x, wv[j].x, acc[i][j]);
          acc[i][j] = fmaf(xv[i].y, wv[j].y, acc[i][j]);
          acc[i][j] = fmaf(xv[i].z, wv[j].z, acc[i][j]);
          acc[i][j] = fmaf(xv[i].w, wv[j].w, acc[i][j]);
        }
    };
    if (cn == CK) {
      // whole tile: unrolled, so the LDS reads run ahead of the fma chains
#pragma unroll
      for (int cc = 0; cc < CK; cc += 4) step(cc);
    } else {
      for (int cc = 0; cc < cn; cc += 4) step(cc);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      const int64_t t = t0 + tok + 8 * i;
      const int e = e0 + el + 32 * j;
      if (t >= ntok || e >= E) continue;
      float v = acc[i][j];
      if (bias) v = v + bias[e];
      if (noise) v = v + noise[t * E + e];
      logits[t * E + e] = v;
    }
}

// ------------------------------------------------------------------ top-k
//
// A group of G = min(32, pow2ceil(E)) lanes (64 past 512 experts) serves one
// token; a wave serves 64/G tokens.  Lane s of a group holds experts s, s+G,
// s+2G, ...  Each of the
// k rounds takes the best unselected value of every lane and reduces it over
// the group with xor-shuffles (greater value wins; equal values -> lower id).
// The winner of round j is kept by lane j of the group.
constexpr int kMaxPerLane = kMaxExperts / 64;   // 16

// A total order: greater value first, equal values (-0 == +0) by lower id,
// and a NaN below every number (NaNs among themselves by lower id), so every
// lane of a group agrees on each round's winner whatever the logits hold.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  const bool na = va != va, nb = vb != vb;
  if (na || nb) return nb && (!na || ia < ib);
  return va > vb || (va == vb && ia < ib);
}

// With a selection bias (nullable) the compared value is the fp32 sum
// logit + sel_bias[e]; the softmax always takes the selected logits alone.
// VPL: experts per lane, ceil(E / G) rounded up to a power of two.
template <int G, int VPL>
__global__ __launch_bounds__(256) void k_route(const float *__restrict__ logits,
                                               const float *__restrict__ sel_bias, int64_t ntok,
                                               int E, int k, int32_t *__restrict__ topk_idx,
                                               float *__restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int s = lane % G;
  const int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) / G;
  const bool live = t < ntok;
  static_assert(VPL >= 1 && VPL <= kMaxPerLane, "experts per lane");
  const int vpl = (E + G - 1) / G;
  float val[VPL];
  unsigned taken = 0u;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = s + v * G;
    const bool ok = v < vpl && e < E;
    val[v] = (live && ok) ? logits[t * E + e] : 0.0f;
    if (sel_bias && ok) val[v] += sel_bias[e];
    if (!ok) taken |= 1u << v;   // padding never wins
  }
  float my_val = 0.0f;
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      if (taken & (1u << v)) continue;
      const int e = s + v * G;
      if (bi == 0x7fffffff || better(val[v], e, bv, bi)) {
        bv = val[v];
        bi = e;
      }
    }
#pragma unroll
    for (int m = 1; m < G; m <<= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oi = __shfl_xor(bi, m, 64);
      if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi % G == s) taken |= 1u << (bi / G);
    if (s == j) {
      my_val = bv;
      my_idx = bi;
    }
  }
  // softmax over the k selected logits, shifted by their maximum (without a
  // selection bias that is the first selected value)
  if (sel_bias && live && s < k) my_val = logits[t * E + my_idx];
  float mx = (s < k) ? my_val : -INFINITY;
#pragma unroll
  for (int m = 1; m < G; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  float ex = (s < k) ? __expf(my_val - mx) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int m = 1; m < G; m <<= 1) sum += __shfl_xor(sum, m, 64);
  if (live && s < k) {
    topk_idx[t * k + s] = my_idx;
    topk_w[t * k + s] = ex / sum;
  }
}

// ------------------------------------------------------------------ route bwd
//
// Same grouping.  Lane j < k holds selection j: g_j = d_row_scale at its row,
// w_j.  S = sum_i w_i g_i by a fixed xor-butterfly; each lane then writes the
// experts it owns: w_j (g_j - S) if selected, else 0.
template <int G>
__global__ __launch_bounds__(256) void k_route_bwd(const int32_t *__restrict__ topk_idx,
                                                   const float *__restrict__ topk_w,
                                                   const float *__restrict__ d_row_scale,
                                                   const int32_t *__restrict__ slot_to_row,
                                                   int64_t ntok, int E, int k,
                                                   float *__restrict__ d_topk_w,
                                                   float *__restrict__ d_logits) {
  const int lane = threadIdx.x & 63;
  const int s = lane % G;
  const int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) / G;
  const bool live = t < ntok;
  int idx = -1;
  float w = 0.0f, g = 0.0f;
  if (live && s < k) {
    const int64_t slot = t * k + s;
    idx = topk_idx[slot];
    w = topk_w[slot];
    const int row = slot_to_row[slot];
    g = row >= 0 ? d_row_scale[row] : 0.0f;   // a dropped slot has no row
    if (d_topk_w) d_topk_w[slot] = g;
  }
  float S = w * g;
#pragma unroll
  for (int m = 1; m < G; m <<= 1) S += __shfl_xor(S, m, 64);
  const float dl = w * (g - S);
  const int base = lane - s;   // first lane of the group
  const int vpl = (E + G - 1) / G;
  for (int v = 0; v < vpl; ++v) {
    const int e = s + v * G;
    float out = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int ij = __shfl(idx, base + j, 64);
      const float dj = __shfl(dl, base + j, 64);
      if (ij == e) out = dj;
    }
    if (live && e < E) d_logits[t * E + e] = out;
  }
}

// ------------------------------------------------------------------ router bwd
//
// dx_router[t,:] = sum_e d_logits[t,e] * w_r[e,:] (e ascending, fp32 fma;
// terms with d_logits == 0 are skipped, they add exact zeros).  One block per
// token, each thread owns runs of 8 columns (16-byte loads and stores).
template <typename T>
__global__ __launch_bounds__(256) void k_router_dx(const float *__restrict__ d_logits,
                                                   const T *__restrict__ wr, int64_t ntok, int d,
                                                   int E, float *__restrict__ dx) {
  const int64_t t = blockIdx.x;
  const float *dl = d_logits + t * E;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int e = 0; e < E; ++e) {
      const float a = dl[e];
      if (a == 0.0f) continue;
      Raw8 r;
      load8_raw(wr + (int64_t)e * d + c, r);
      float w[8];
      widen8<T>(r, w);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(a, w[i], acc[i]);
    }
    float4 *out = reinterpret_cast<float4 *>(dx + t * d + c);
    out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

// dw_r partials: block (e, column tile of 2048, token chunk of 256).  The
// nonzero entries of d_logits[:,e] inside the chunk are found with a ballot
// and visited in token order; each thread owns 8 consecutive columns.
constexpr int kDwTokChunk = 256;
constexpr int kDwCols = 2048;

template <typename T>
__global__ __launch_bounds__(256) void k_router_dw_partial(const float *__restrict__ d_logits,
                                                           const T *__restrict__ x, int64_t ntok,
                                                           int d, int E,
                                                           float *__restrict__ partial) {
  const int e = blockIdx.z;
  const int chunk = blockIdx.y;
  const int c = blockIdx.x * kDwCols + threadIdx.x * 8;
  const int64_t tbeg = (int64_t)chunk * kDwTokChunk;
  __shared__ int s_tok[kDwTokChunk];
  __shared__ float s_val[kDwTokChunk];
  __shared__ int s_cnt[4];
  // compact the nonzero entries of this chunk, keeping token order
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NI = kDwTokChunk / 256;   // 64-token groups per wave
  int nz[NI];
  float vals[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {   // wave w scans tokens [w*64*NI, (w+1)*64*NI)
    const int64_t t = tbeg + wave * 64 * NI + i * 64 + lane;
    const float v = (t < ntok) ? d_logits[t * E + e] : 0.0f;
    vals[i] = v;
    nz[i] = v != 0.0f;
  }
  int wave_tot = 0;
  int pos[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint64_t m = __ballot(nz[i]);
    pos[i] = wave_tot + __popcll(m & ((1ull << lane) - 1ull));
    wave_tot += __popcll(m);
  }
  if (lane == 0) s_cnt[wave] = wave_tot;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += s_cnt[w];
  const int total = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (nz[i]) {
      s_tok[wbase + pos[i]] = (int)(wave * 64 * NI + i * 64 + lane);
      s_val[wbase + pos[i]] = vals[i];
    }
  }
  __syncthreads();
  if (c < d) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    // four rows' loads in flight, then their fmas in token order
    int n = 0;
    for (; n + 4 <= total; n += 4) {
      Raw8 r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) load8_raw(x + (tbeg + s_tok[n + u]) * d + c, r[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float a = s_val[n + u];
        float xv[8];
        widen8<T>(r[u], xv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(a, xv[i], acc[i]);
      }
    }
    for (; n < total; ++n) {
      const int64_t t = tbeg + s_tok[n];
      const float a = s_val[n];
      Raw8 r;
      load8_raw(x + t * d + c, r);
      float xv[8];
      widen8<T>(r, xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(a, xv[i], acc[i]);
    }
    float4 *out = reinterpret_cast<float4 *>(partial + ((int64_t)e * gridDim.y + chunk) * d + c);
    out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

__global__ __launch_bounds__(256) void k_router_dw_reduce(const float *__restrict__ partial,
                                                          int nchunk, int d, int E,
                                                          float *__restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)E * d) return;
  const int64_t e = i / d, c = i % d;
  const float *p = partial + e * nchunk * d + c;
  // eight chunks' loads in flight, summed in chunk order
  float s = 0.0f;
  int ch = 0;
  for (; ch + 8 <= nchunk; ch += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(ch + u) * d];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; ch < nchunk; ++ch) s += p[(int64_t)ch * d];
  dw[i] = s;
}

__global__ __launch_bounds__(256) void k_fill_zero(float *__restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

}  // namespace moe

using namespace moe;

// ====================================================================== C ABI

static int check_common(int64_t T, int E, const char *fn) {
  MOE_REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "%s: T < 0", fn);
  MOE_REQUIRE(E >= 1 && E <= kMaxExperts, MOE_ERR_UNSUPPORTED, "%s: E=%d outside [1,%d]", fn, E,
              kMaxExperts);
  return MOE_OK;
}

extern "C" int moe_router_logits(const void *x, const void *w_r, const float *bias,
                                 const float *logit_add, int dtype, int64_t T, int d, int E,
                                 float *logits, void *stream) {
  clear_error();
  int rc = check_common(T, E, "moe_router_logits");
  if (rc) return rc;
  MOE_REQUIRE(dtype == MOE_BF16 || dtype == MOE_F32, MOE_ERR_UNSUPPORTED,
              "moe_router_logits: dtype %d", dtype);
  MOE_REQUIRE(d > 0 && d % 8 == 0, MOE_ERR_UNSUPPORTED, "moe_router_logits: d=%d", d);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(x && w_r && logits, MOE_ERR_INVALID_ARG, "moe_router_logits: null pointer");
  MOE_REQUIRE(aligned16(x) && aligned16(w_r) && aligned16(logits), MOE_ERR_INVALID_ARG,
              "moe_router_logits: pointers must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  // blocked chains once there are enough of them to keep every SIMD busy
  // (measured: at T*E = 2^17, two tokens per lane ran 45 against 39 us)
  const bool many = T * (int64_t)E >= ((int64_t)1 << 20);
  const int TB = many ? (E > kLogitExp ? 2 : 4) : 1, EB = many && E > kLogitExp ? 2 : 1;
  dim3 grid((unsigned)((T + kLogitTok * TB - 1) / (kLogitTok * TB)),
            (unsigned)((E + kLogitExp * EB - 1) / (kLogitExp * EB)));
#define LOGITS_CASE(TT, TBV, EBV)                                                             \
  MOE_LAUNCH("router_logits", s,                                                              \
             (k_router_logits<TT, TBV, EBV><<<grid, 256, 0, s>>>(                               \
                 (const TT *)x, (const TT *)w_r, bias, logit_add, T, d, E, logits)))
  if (dtype == MOE_BF16) {
    if (TB == 1) LOGITS_CASE(bf16_t, 1, 1);
    else if (EB == 2) LOGITS_CASE(bf16_t, 2, 2);
    else LOGITS_CASE(bf16_t, 4, 1);
  } else {
    if (TB == 1) LOGITS_CASE(float, 1, 1);
    else if (EB == 2) LOGITS_CASE(float, 2, 2);
    else LOGITS_CASE(float, 4, 1);
  }
#undef LOGITS_CASE
  return check_launch("moe_router_logits");
}

static int route_impl(const float *logits, const float *sel_bias, int64_t T, int E, int k,
                      int32_t *topk_idx, float *topk_w, void *stream, const char *fn) {
  clear_error();
  int rc = check_common(T, E, fn);
  if (rc) return rc;
  MOE_REQUIRE(k >= 1 && k <= E && k <= kMaxTopK, MOE_ERR_UNSUPPORTED, "%s: k=%d E=%d", fn, k, E);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(logits && topk_idx && topk_w, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  hipStream_t s = (hipStream_t)stream;
  // Groups of up to 32 lanes (64 past 512 experts, at most 16 experts per
  // lane): each round's reduction then takes one xor step fewer and a wave
  // serves two tokens.
  const int gmax = E > 32 * kMaxPerLane ? 64 : 32;
  int G = 1;
  while (G < E && G < gmax) G <<= 1;
  const int64_t threads = T * G;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  const char *name = sel_bias ? "route_topk_biased" : "route_topk";
  int vpl = 1;   // experts per lane of a group, a power of two
  while (vpl * G < E) vpl <<= 1;
#define ROUTE_CASE(GV, VV)                                                                    \
  MOE_LAUNCH(name, s,                                                                         \
             (k_route<GV, VV><<<blocks, 256, 0, s>>>(logits, sel_bias, T, E, k, topk_idx,      \
                                                     topk_w)))
  switch (G) {
    case 1: ROUTE_CASE(1, 1); break;
    case 2: ROUTE_CASE(2, 1); break;
    case 4: ROUTE_CASE(4, 1); break;
    case 8: ROUTE_CASE(8, 1); break;
    case 16: ROUTE_CASE(16, 1); break;
    case 32:
      switch (vpl) {
        case 1: ROUTE_CASE(32, 1); break;
        case 2: ROUTE_CASE(32, 2); break;
        case 4: ROUTE_CASE(32, 4); break;
        case 8: ROUTE_CASE(32, 8); break;
        default: ROUTE_CASE(32, 16); break;
      }
      break;
    default:
      switch (vpl) {
        case 1: ROUTE_CASE(64, 1); break;
        case 2: ROUTE_CASE(64, 2); break;
        case 4: ROUTE_CASE(64, 4); break;
        case 8: ROUTE_CASE(64, 8); break;
        default: ROUTE_CASE(64, 16); break;
      }
  }
#undef ROUTE_CASE
  return check_launch(fn);
}

extern "C" int moe_route(const float *logits, int64_t T, int E, int k, int32_t *topk_idx,
                         float *topk_w, void *stream) {
  return route_impl(logits, nullptr, T, E, k, topk_idx, topk_w, stream, "moe_route");
}

extern "C" int moe_route_biased(const float *logits, const float *sel_bias, int64_t T, int E,
                                int k, int32_t *topk_idx, float *topk_w, void *stream) {
  if (!sel_bias && T > 0) {
    clear_error();
    MOE_REQUIRE(false, MOE_ERR_INVALID_ARG, "moe_route_biased: null sel_bias");
  }
  return route_impl(logits, sel_bias, T, E, k, topk_idx, topk_w, stream, "moe_route_biased");
}

extern "C" int moe_route_bwd(const int32_t *topk_idx, const float *topk_w,
                             const float *d_row_scale, const int32_t *slot_to_row, int64_t T,
                             int E, int k, float *d_topk_w, float *d_logits, void *stream) {
  clear_error();
  int rc = check_common(T, E, "moe_route_bwd");
  if (rc) return rc;
  MOE_REQUIRE(k >= 1 && k <= E && k <= kMaxTopK, MOE_ERR_UNSUPPORTED, "moe_route_bwd: k=%d E=%d",
              k, E);
  MOE_REQUIRE((int64_t)T * k < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED, "moe_route_bwd: T*k too big");
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(topk_idx && topk_w && d_row_scale && slot_to_row && d_logits, MOE_ERR_INVALID_ARG,
              "moe_route_bwd: null pointer");
  hipStream_t s = (hipStream_t)stream;
  int G = 1;
  while (G < E && G < 64) G <<= 1;
  const unsigned blocks = (unsigned)((T * G + 255) / 256);
#define RB_CASE(GV)                                                                             \
  case GV:                                                                                      \
    MOE_LAUNCH("route_bwd", s,                                                                  \
               k_route_bwd<GV><<<blocks, 256, 0, s>>>(topk_idx, topk_w, d_row_scale, slot_to_row, \
                                                      T, E, k, d_topk_w, d_logits));            \
    break
  switch (G) {
    RB_CASE(1); RB_CASE(2); RB_CASE(4); RB_CASE(8); RB_CASE(16); RB_CASE(32); RB_CASE(64);
  }
#undef RB_CASE
  return check_launch("moe_route_bwd");
}

extern "C" size_t moe_router_logits_bwd_workspace_size(int64_t T, int d, int E) {
  if (T <= 0 || d <= 0 || E <= 0) return 256;
  const int64_t nchunk = (T + kDwTokChunk - 1) / kDwTokChunk;
  return align_up((size_t)E * (size_t)nchunk * (size_t)d * sizeof(float), 256);
}

extern "C" int moe_router_logits_bwd(const void *x, const void *w_r, const float *d_logits,
                                     int dtype, int64_t T, int d, int E, float *dx_router,
                                     float *dw_r, void *ws, size_t ws_bytes, void *stream) {
  clear_error();
  int rc = check_common(T, E, "moe_router_logits_bwd");
  if (rc) return rc;
  MOE_REQUIRE(dtype == MOE_BF16 || dtype == MOE_F32, MOE_ERR_UNSUPPORTED,
              "moe_router_logits_bwd: dtype %d", dtype);
  MOE_REQUIRE(d > 0 && d % 8 == 0 && d <= 65536, MOE_ERR_UNSUPPORTED, "moe_router_logits_bwd: d=%d", d);
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {
    if (dw_r) {
      MOE_REQUIRE(aligned16(dw_r), MOE_ERR_INVALID_ARG, "moe_router_logits_bwd: dw_r alignment");
      const int64_t n = (int64_t)E * d;
      MOE_LAUNCH("router_dw_zero", s,
                 k_fill_zero<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(dw_r, n));
      return check_launch("moe_router_logits_bwd(zero)");
    }
    return MOE_OK;
  }
  MOE_REQUIRE(d_logits, MOE_ERR_INVALID_ARG, "moe_router_logits_bwd: null d_logits");
  if (dx_router) {
    MOE_REQUIRE(w_r && aligned16(w_r) && aligned16(dx_router), MOE_ERR_INVALID_ARG,
                "moe_router_logits_bwd: w_r / dx_router");
    const unsigned blocks = (unsigned)T;
    if (dtype == MOE_BF16)
      MOE_LAUNCH("router_dx", s,
                 k_router_dx<bf16_t><<<blocks, 256, 0, s>>>(d_logits, (const bf16_t *)w_r, T, d, E,
                                                            dx_router));
    else
      MOE_LAUNCH("router_dx", s,
                 k_router_dx<float><<<blocks, 256, 0, s>>>(d_logits, (const float *)w_r, T, d, E,
                                                           dx_router));
    rc = check_launch("moe_router_logits_bwd(dx)");
    if (rc) return rc;
  }
  if (dw_r) {
    MOE_REQUIRE(x && aligned16(x) && aligned16(dw_r), MOE_ERR_INVALID_ARG,
                "moe_router_logits_bwd: x / dw_r");
    const size_t need = moe_router_logits_bwd_workspace_size(T, d, E);
    MOE_REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE,
                "moe_router_logits_bwd: workspace %zu < %zu", ws_bytes, need);
    const int nchunk = (int)((T + kDwTokChunk - 1) / kDwTokChunk);
    dim3 grid((unsigned)((d + kDwCols - 1) / kDwCols), (unsigned)nchunk, (unsigned)E);
    float *partial = (float *)ws;
    if (dtype == MOE_BF16)
      MOE_LAUNCH("router_dw_partial", s,
                 k_router_dw_partial<bf16_t><<<grid, 256, 0, s>>>(d_logits, (const bf16_t *)x, T,
                                                                  d, E, partial));
    else
      MOE_LAUNCH("router_dw_partial", s,
                 k_router_dw_partial<float><<<grid, 256, 0, s>>>(d_logits, (const float *)x, T, d,
                                                                 E, partial));
    rc = check_launch("moe_router_logits_bwd(dw partial)");
    if (rc) return rc;
    const unsigned rblocks = (unsigned)(((int64_t)E * d + 255) / 256);
    MOE_LAUNCH("router_dw_reduce", s,
               k_router_dw_reduce<<<rblocks, 256, 0, s>>>(partial, nchunk, d, E, dw_r));
    rc = check_launch("moe_router_logits_bwd(dw reduce)");
    if (rc) return rc;
  }
  return MOE_OK;
}
