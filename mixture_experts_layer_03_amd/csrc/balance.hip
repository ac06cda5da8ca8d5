// Expert-load statistics over a valid token prefix, the selection-bias
// balancing update, and the load-balancing auxiliary loss with its gradient.
//
// The pages name three router features without formulas: balancing through an
// expert-selection bias for a family that has no router auxiliary loss ("Halo's
// 2.8x over TRL is not a kernel, and its own benchmark proves it", section "The
// small-hardware end", the LFM2 config and the paragraph after it); a router
// auxiliary loss with a per-run coefficient whose gradient the routers apply
// while reporting the unscaled and scaled values (the TorchTurbo page,
// "inclusionAI open-sources TorchTurbo, a SuperNode-native post-training
// engine", section "Adapter", ms-swift DPO); and MoE statistics that skip the
// right-padded tail of a batch (same TorchTurbo page, section "Model",
// sequence-parallel input contract).  Readings used here:
//   load_e      = #{(t, j) : t < n_valid, topk_idx[t,j] = e}
//   bias update : b_e += rate * sign(n_valid * k / E - load_e)
//   aux         = E * sum_e (load_e / (n_valid k)) * P_e,
//                 P_e = (1/n_valid) sum_{t < n_valid} softmax(L[t,:])_e
//   d aux_scaled / d L[t,e] = p_te (g_e - sum_e' p_te' g_e'),
//                 g_e = coeff * E * load_e / (n_valid^2 k), t < n_valid only.
//
// All reductions run in a fixed order (per-block partials, then one ordered
// pass), so results do not depend on scheduling; the counts are exact.
#include "moe_internal.h"

namespace moe {

constexpr int kLoadChunk = 2048;     // slots per block of the load histogram
constexpr int kAuxMaxPasses = 8;     // token passes per block of the aux kernel
constexpr int kAuxTargetBlocks = 2048;   // enough resident blocks to hide latency
constexpr int kAuxMaxPerLane = kMaxExperts / 64;

// Per-block histogram of the first nslots slots into part[block][E].
__global__ __launch_bounds__(256) void k_load_partial(const int32_t *__restrict__ idx,
                                                      int64_t nslots, int E,
                                                      int32_t *__restrict__ part) {
  __shared__ int h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t beg = (int64_t)blockIdx.x * kLoadChunk;
  const int64_t end = min(beg + (int64_t)kLoadChunk, nslots);
  if (end - beg == kLoadChunk && (reinterpret_cast<uintptr_t>(idx) & 15u) == 0) {
    // full chunk: both 16-byte loads of a thread are issued before any count
    static_assert(kLoadChunk == 256 * 8, "two int4 per thread");
    const int4 *v = reinterpret_cast<const int4 *>(idx + beg);
    const int4 a = v[threadIdx.x], b = v[threadIdx.x + 256];
    const int ids[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (ids[i] >= 0 && ids[i] < E) atomicAdd(&h[ids[i]], 1);   // LDS integer adds
  } else {
    for (int64_t s = beg + threadIdx.x; s < end; s += 256) {
      const int e = idx[s];
      if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) part[(int64_t)blockIdx.x * E + e] = h[e];
}

// Column sums of a [rows, E] table of per-block partials: a block of
// kColWaves waves covers 64 experts (lane = expert, so each row's read is
// one coalesced line per wave) and rows [y*kColRows, (y+1)*kColRows); wave w
// takes the rows w, w + kColWaves, ... ascending, and the waves' sums are
// added in wave order.  The order is fixed by the shape alone.
constexpr int kColWaves = 16, kColRows = 256;

template <typename T>
__device__ __forceinline__ T col_sum(const T *__restrict__ tab, int rows, int E, int e, int y,
                                     int w) {
  const int r0 = y * kColRows, r1 = min(rows, r0 + kColRows);
  T acc = T(0);
  int r = r0 + w;
  // four rows' loads in flight per lane, added in row order
  for (; r + 3 * kColWaves < r1; r += 4 * kColWaves) {
    T v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = e < E ? tab[(int64_t)(r + u * kColWaves) * E + e] : T(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += v[u];
  }
  for (; r < r1; r += kColWaves) acc += e < E ? tab[(int64_t)r * E + e] : T(0);
  return acc;
}

// load[e] = sum over blocks of part[b][e] (integer counts: exact).
__global__ __launch_bounds__(kColWaves * 64) void k_load_reduce(const int32_t *__restrict__ part,
                                                                int nblk, int E,
                                                                int32_t *__restrict__ load) {
  __shared__ int red[kColWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  int c = 0;
  for (int y = 0; y * kColRows < nblk; ++y) c += col_sum<int32_t>(part, nblk, E, e, y, w);
  red[w][lane] = c;
  __syncthreads();
  if (w == 0 && e < E) {
    int t = 0;
    for (int i = 0; i < kColWaves; ++i) t += red[i][lane];
    load[e] = t;
  }
}

// b_e + rate * sign(n_valid*k - E*load_e): the sign is an exact integer
// comparison; one fp32 add per expert (a zero step still adds +0).
__global__ __launch_bounds__(256) void k_bias_update(const int32_t *__restrict__ load,
                                                     int64_t nk, int E, float rate,
                                                     float *__restrict__ sel_bias) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const int64_t diff = nk - (int64_t)E * load[e];
  const float step = diff > 0 ? rate : (diff < 0 ? -rate : 0.0f);
  sel_bias[e] = sel_bias[e] + step;
}

// Token-group layout of the router kernels: G lanes per token (G = the power
// of two >= E, at most 64), lane s owns experts s, s+G, ...  Each block takes
// passes * (256/G) consecutive tokens below n_valid (passes chosen on the host
// so that the grid has about kAuxTargetBlocks blocks).  Per token: the full
// softmax p (max-shifted, fp32), the running per-expert sum of p, and (if
// d_logits is given) the gradient added into d_logits.  At the end the token
// groups' sums are combined in group order into psum[block][E].
template <int G>
__global__ __launch_bounds__(256) void k_aux_partial(const float *__restrict__ logits,
                                                     const int32_t *__restrict__ load,
                                                     int64_t n_valid, int E, int passes,
                                                     float gscale, float *__restrict__ d_logits,
                                                     float *__restrict__ psum) {
  constexpr int kGroups = 256 / G;
  __shared__ float red[kGroups * kAuxMaxPerLane * G];
  const int s = threadIdx.x % G;
  const int grp = threadIdx.x / G;
  const int vpl = (E + G - 1) / G;
  float acc[kAuxMaxPerLane], g[kAuxMaxPerLane];
#pragma unroll
  for (int v = 0; v < kAuxMaxPerLane; ++v) {
    const int e = s + v * G;
    acc[v] = 0.0f;
    g[v] = (v < vpl && e < E) ? gscale * (float)load[e] : 0.0f;
  }
  const int64_t t0 = (int64_t)blockIdx.x * passes * kGroups;
  for (int pass = 0; pass < passes; ++pass) {
    const int64_t t = t0 + (int64_t)pass * kGroups + grp;
    if (t >= n_valid) break;   // the same for every lane of the group
    float val[kAuxMaxPerLane];
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < kAuxMaxPerLane; ++v) {
      const int e = s + v * G;
      const bool ok = v < vpl && e < E;
      val[v] = ok ? logits[t * E + e] : -INFINITY;
      mx = fmaxf(mx, val[v]);
    }
#pragma unroll
    for (int m = 1; m < G; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
    float z = 0.0f;
#pragma unroll
    for (int v = 0; v < kAuxMaxPerLane; ++v) {
      const int e = s + v * G;
      val[v] = (v < vpl && e < E) ? __expf(val[v] - mx) : 0.0f;
      z += val[v];
    }
#pragma unroll
    for (int m = 1; m < G; m <<= 1) z += __shfl_xor(z, m, 64);
    const float rz = 1.0f / z;
    float pg = 0.0f;
#pragma unroll
    for (int v = 0; v < kAuxMaxPerLane; ++v) {
      val[v] *= rz;
      acc[v] += val[v];
      pg += val[v] * g[v];
    }
    if (d_logits) {
#pragma unroll
      for (int m = 1; m < G; m <<= 1) pg += __shfl_xor(pg, m, 64);
#pragma unroll
      for (int v = 0; v < kAuxMaxPerLane; ++v) {
        const int e = s + v * G;
        if (v < vpl && e < E) {
          float *q = d_logits + t * E + e;
          *q = *q + val[v] * (g[v] - pg);
        }
      }
    }
  }
#pragma unroll
  for (int v = 0; v < kAuxMaxPerLane; ++v)
    if (v < vpl) red[(grp * kAuxMaxPerLane + v) * G + s] = acc[v];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    const int v = e / G, ls = e % G;
    float sum = 0.0f;
    for (int q = 0; q < kGroups; ++q) sum += red[(q * kAuxMaxPerLane + v) * G + ls];
    psum[(int64_t)blockIdx.x * E + e] = sum;
  }
}

// Psum partials: pcol[y][e] = sum of psum[b][e] over the rows of row block
// y (col_sum's order), grid (ceil(E/64), ceil(nblk/kColRows)).
__global__ __launch_bounds__(kColWaves * 64) void k_aux_colsum(const float *__restrict__ psum,
                                                               int nblk, int E,
                                                               float *__restrict__ pcol) {
  __shared__ float red[kColWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  red[w][lane] = col_sum<float>(psum, nblk, E, e, blockIdx.y, w);
  __syncthreads();
  if (w == 0 && e < E) {
    float t = 0.0f;
    for (int i = 0; i < kColWaves; ++i) t += red[i][lane];
    pcol[(int64_t)blockIdx.y * E + e] = t;
  }
}

// One block of 1024 threads.  Psum_e = sum over the row blocks y (ascending)
// of pcol[y][e], then sum_e load_e * Psum_e by a fixed tree, aux = that * E /
// (n_valid^2 k); out[0] = aux, out[1] = coeff * aux.
__global__ __launch_bounds__(1024) void k_aux_final(const float *__restrict__ pcol, int ny,
                                                    const int32_t *__restrict__ load, int E,
                                                    float norm, float coeff,
                                                    float *__restrict__ out) {
  __shared__ float red[1024];
  const int tid = threadIdx.x;
  float term = 0.0f;
  if (tid < E) {
    float P = 0.0f;
    for (int y = 0; y < ny; ++y) P += pcol[(int64_t)y * E + tid];
    term = (float)load[tid] * P;
  }
  red[tid] = term;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float aux = red[0] * norm;
    out[0] = aux;
    out[1] = coeff * aux;
  }
}

__global__ __launch_bounds__(64) void k_aux_zero(float *__restrict__ out) {
  if (threadIdx.x < 2) out[threadIdx.x] = 0.0f;
}

static int route_group(int E) {
  int G = 1;
  while (G < E && G < 64) G <<= 1;
  return G;
}

static int64_t load_blocks(int64_t nslots) { return (nslots + kLoadChunk - 1) / kLoadChunk; }

// token passes per block: 1 until the grid would exceed kAuxTargetBlocks
static int aux_passes(int64_t n_valid, int E) {
  const int64_t groups = 256 / route_group(E);
  const int64_t blocks1 = (n_valid + groups - 1) / groups;
  int64_t p = blocks1 / kAuxTargetBlocks;
  return (int)(p < 1 ? 1 : (p > kAuxMaxPasses ? kAuxMaxPasses : p));
}

static int64_t aux_blocks(int64_t n_valid, int E) {
  const int64_t per = (int64_t)aux_passes(n_valid, E) * (256 / route_group(E));
  return (n_valid + per - 1) / per;
}

}  // namespace moe

using namespace moe;

// ====================================================================== C ABI

static int check_stats_args(int64_t T, int64_t n_valid, int E, int k, const char *fn) {
  MOE_REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "%s: T < 0", fn);
  MOE_REQUIRE(n_valid >= 0 && n_valid <= T, MOE_ERR_INVALID_ARG,
              "%s: n_valid=%lld outside [0, T=%lld]", fn, (long long)n_valid, (long long)T);
  MOE_REQUIRE(E >= 1 && E <= kMaxExperts, MOE_ERR_UNSUPPORTED, "%s: E=%d outside [1,%d]", fn, E,
              kMaxExperts);
  MOE_REQUIRE(k >= 1 && k <= E && k <= kMaxTopK, MOE_ERR_UNSUPPORTED, "%s: k=%d E=%d", fn, k, E);
  MOE_REQUIRE(T * (int64_t)k < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED, "%s: T*k too big", fn);
  return MOE_OK;
}

extern "C" size_t moe_expert_load_workspace_size(int64_t T, int E, int k) {
  if (T <= 0 || E <= 0 || k <= 0) return 256;
  return align_up((size_t)load_blocks(T * (int64_t)k) * (size_t)E * sizeof(int32_t), 256);
}

extern "C" int moe_expert_load(const int32_t *topk_idx, int64_t T, int64_t n_valid, int E, int k,
                               int32_t *load, void *ws, size_t ws_bytes, void *stream) {
  clear_error();
  int rc = check_stats_args(T, n_valid, E, k, "moe_expert_load");
  if (rc) return rc;
  MOE_REQUIRE(load, MOE_ERR_INVALID_ARG, "moe_expert_load: null load");
  const int64_t nslots = n_valid * k;
  const int64_t nblk = load_blocks(nslots);
  if (nblk > 0) {
    MOE_REQUIRE(topk_idx && ws, MOE_ERR_INVALID_ARG, "moe_expert_load: null pointer");
    MOE_REQUIRE(ws_bytes >= (size_t)nblk * (size_t)E * sizeof(int32_t), MOE_ERR_WORKSPACE,
                "moe_expert_load: workspace %zu < %zu", ws_bytes,
                (size_t)nblk * (size_t)E * sizeof(int32_t));
  }
  hipStream_t s = (hipStream_t)stream;
  int32_t *part = (int32_t *)ws;
  if (nblk > 0)
    MOE_LAUNCH("expert_load", s,
               k_load_partial<<<(unsigned)nblk, 256, 0, s>>>(topk_idx, nslots, E, part));
  MOE_LAUNCH("expert_load_reduce", s,
             k_load_reduce<<<(unsigned)((E + 63) / 64), kColWaves * 64, 0, s>>>(part, (int)nblk, E,
                                                                              load));
  return check_launch("moe_expert_load");
}

extern "C" int moe_bias_update(const int32_t *load, int64_t n_valid, int E, int k, float rate,
                               float *sel_bias, void *stream) {
  clear_error();
  int rc = check_stats_args(n_valid, n_valid, E, k, "moe_bias_update");
  if (rc) return rc;
  MOE_REQUIRE(load && sel_bias, MOE_ERR_INVALID_ARG, "moe_bias_update: null pointer");
  MOE_REQUIRE(rate == rate && rate >= 0.0f && rate < INFINITY, MOE_ERR_INVALID_ARG,
              "moe_bias_update: rate must be finite and >= 0");
  hipStream_t s = (hipStream_t)stream;
  MOE_LAUNCH("bias_update", s,
             k_bias_update<<<(unsigned)((E + 255) / 256), 256, 0, s>>>(load, n_valid * k, E, rate,
                                                                     sel_bias));
  return check_launch("moe_bias_update");
}

// The per-block sums psum[nblk][E], then the row-block sums pcol[ny][E].
static size_t aux_psum_bytes(int64_t nblk, int E) {
  return align_up((size_t)nblk * (size_t)E * sizeof(float), 256);
}
static size_t aux_pcol_bytes(int64_t nblk, int E) {
  return align_up((size_t)((nblk + kColRows - 1) / kColRows) * (size_t)E * sizeof(float), 256);
}

// Sized for one pass per block, which bounds the grid of every n_valid <= T.
extern "C" size_t moe_aux_loss_workspace_size(int64_t T, int E) {
  if (T <= 0 || E <= 0 || E > kMaxExperts) return 256;
  const int64_t groups = 256 / route_group(E);
  const int64_t nmax = (T + groups - 1) / groups;
  return aux_psum_bytes(nmax, E) + aux_pcol_bytes(nmax, E);
}

extern "C" int moe_aux_loss(const float *logits, const int32_t *load, int64_t T, int64_t n_valid,
                            int E, int k, float coeff, float *aux_out, float *d_logits, void *ws,
                            size_t ws_bytes, void *stream) {
  clear_error();
  int rc = check_stats_args(T, n_valid, E, k, "moe_aux_loss");
  if (rc) return rc;
  MOE_REQUIRE(aux_out, MOE_ERR_INVALID_ARG, "moe_aux_loss: null aux_out");
  MOE_REQUIRE(coeff == coeff && coeff > -INFINITY && coeff < INFINITY, MOE_ERR_INVALID_ARG,
              "moe_aux_loss: coeff must be finite");
  hipStream_t s = (hipStream_t)stream;
  if (n_valid == 0) {
    MOE_LAUNCH("aux_loss_final", s, k_aux_zero<<<1, 64, 0, s>>>(aux_out));
    return check_launch("moe_aux_loss");
  }
  MOE_REQUIRE(logits && load && ws, MOE_ERR_INVALID_ARG, "moe_aux_loss: null pointer");
  const int64_t nblk = aux_blocks(n_valid, E);
  const int passes = aux_passes(n_valid, E);
  const size_t need = aux_psum_bytes(nblk, E) + aux_pcol_bytes(nblk, E);
  MOE_REQUIRE(ws_bytes >= need, MOE_ERR_WORKSPACE, "moe_aux_loss: workspace %zu < %zu", ws_bytes,
              need);
  const double n = (double)n_valid;
  const float gscale = (float)((double)coeff * E / (n * n * k));
  const float norm = (float)((double)E / (n * n * k));
  float *psum = (float *)ws;
  float *pcol = (float *)((char *)ws + aux_psum_bytes(nblk, E));
  const int ny = (int)((nblk + kColRows - 1) / kColRows);
  const int G = route_group(E);
#define AUX_CASE(GV)                                                                          \
  case GV:                                                                                    \
    MOE_LAUNCH("aux_loss", s,                                                                 \
               k_aux_partial<GV><<<(unsigned)nblk, 256, 0, s>>>(logits, load, n_valid, E,      \
                                                                passes, gscale, d_logits,     \
                                                                psum));                       \
    break
  switch (G) {
    AUX_CASE(1); AUX_CASE(2); AUX_CASE(4); AUX_CASE(8); AUX_CASE(16); AUX_CASE(32); AUX_CASE(64);
  }
#undef AUX_CASE
  MOE_LAUNCH("aux_loss_colsum", s,
             k_aux_colsum<<<dim3((unsigned)((E + 63) / 64), (unsigned)ny), kColWaves * 64, 0, s>>>(
                 psum, (int)nblk, E, pcol));
  MOE_LAUNCH("aux_loss_final", s,
             k_aux_final<<<1, 1024, 0, s>>>(pcol, ny, load, E, norm, coeff, aux_out));
  return check_launch("moe_aux_loss");
}
