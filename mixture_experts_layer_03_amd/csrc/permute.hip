// Token permutation into per-expert segments, combine, and their adjoints.
//
// The pages: each expert runs "a grouped matmul over tokens sorted by expert",
// and the rows come back to their token "in the same order, weighted by the
// top-k probabilities" ("Halo's 2.8x over TRL is not a kernel, and its own
// benchmark proves it", section "Where the gap actually is", EP token-routing
// figure).  On one GPU the dispatch all-to-all reduces to this row permutation.
// The backward is written as gathers, with no atomic adds ("Halo: Frontier-Lab
// Training for Everyone", section "Some of the hard problems along the way").
#include "moe_internal.h"

namespace moe {

// ------------------------------------------------------------------ maps
//
// Slots s = t*k + j are cut into chunks of `chunk` consecutive slots.
//  1. k_hist:  per-chunk expert histogram in LDS (integer atomics: the counts
//              do not depend on their order).
//  2. k_scan:  one block scans the histograms in expert-major order, giving
//              every (expert, chunk) its first row, plus counts and offsets.
//  3. k_place: inside a chunk, each wave walks its quarter in slot order,
//              64 slots at a time; the lanes holding the same expert are found
//              with one ballot per expert-id bit, and ranked by lane order.
//              Row = base(expert, chunk) + earlier waves + earlier steps + rank.
// Slots whose expert id is outside [0,E) get no row (slot_to_row = -1).

struct PermPlan {
  int64_t R;
  int nchunk;
  int chunk;   // multiple of 256
};

// Chunks of 256 to 2048 slots: as many as keep the scan's E x nchunk
// histogram within 16384 entries (one block sums them), never fewer than
// 2048-slot chunks give, at most 2048.  k_hist and k_place run one block per
// chunk, each wave of k_place walking its quarter 64 slots at a time, so
// short chunks put more CUs on the maps (16384 slots, 32 experts: 64 chunks
// of 256 instead of 8 of 2048; measured k_place 12.2 -> 6.2 us, k_scan
// 7.1 -> 7.8-8.5 us; at 65536 slots k_place 12.5 -> 6.7, k_scan 7.6 -> 11.0).
static PermPlan perm_plan(int64_t T, int E, int k) {
  PermPlan p;
  p.R = T * k;
  const int64_t by_scan = 16384 / (E > 0 ? E : 1), by_size = (p.R + 2047) / 2048;
  int64_t nchunk = (p.R + 255) / 256;
  if (nchunk > (by_scan > by_size ? by_scan : by_size)) nchunk = by_scan > by_size ? by_scan : by_size;
  if (nchunk > 2048) nchunk = 2048;
  if (nchunk < 1) nchunk = 1;
  int64_t chunk = (p.R + nchunk - 1) / nchunk;
  chunk = (chunk + 255) / 256 * 256;
  if (chunk < 256) chunk = 256;
  p.chunk = (int)chunk;
  p.nchunk = (int)((p.R + chunk - 1) / chunk);
  if (p.nchunk < 1) p.nchunk = 1;
  return p;
}

__global__ __launch_bounds__(256) void k_hist(const int32_t *__restrict__ idx, int64_t R, int E,
                                              int chunk, int nchunk, int32_t *__restrict__ hist) {
  __shared__ int h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t beg = (int64_t)blockIdx.x * chunk;
  const int64_t end = min(beg + chunk, R);
  for (int64_t s = beg + threadIdx.x; s < end; s += 256) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(int64_t)e * nchunk + blockIdx.x] = h[e];
}

// Exclusive scan of n = E*nchunk ints (expert-major) by one block of 1024.
// Each thread sums a contiguous run (eight loads in flight at a time), the
// run sums are scanned in LDS, then each run is rescanned into base[];
// counts come from the per-expert offsets.
__global__ __launch_bounds__(1024) void k_scan(const int32_t *__restrict__ hist, int E, int nchunk,
                                               int32_t *__restrict__ base,
                                               int32_t *__restrict__ counts,
                                               int32_t *__restrict__ offsets) {
  __shared__ int part[1024];
  __shared__ int s_off[kMaxExperts + 1];
  const int64_t n = (int64_t)E * nchunk;
  const int64_t per = (n + 1023) / 1024;
  const int64_t b = threadIdx.x * per;
  const int64_t e_ = min(b + per, n);
  int sum = 0;
  int64_t i = b;
  for (; i + 8 <= e_; i += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = hist[i + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  for (; i < e_; ++i) sum += hist[i];
  part[threadIdx.x] = sum;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partial sums
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = threadIdx.x ? part[threadIdx.x - 1] : 0;
  i = b;
  for (; i + 8 <= e_; i += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = hist[i + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if ((i + u) % nchunk == 0) s_off[(i + u) / nchunk] = run;   // first chunk of an expert
      base[i + u] = run;
      run += v[u];
    }
  }
  for (; i < e_; ++i) {
    if (i % nchunk == 0) s_off[i / nchunk] = run;
    base[i] = run;
    run += hist[i];
  }
  if (threadIdx.x == 1023) s_off[E] = part[1023];
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += 1024) {
    offsets[e] = s_off[e];
    if (e < E) counts[e] = s_off[e + 1] - s_off[e];
  }
}

__device__ __forceinline__ uint64_t peers_of(int e, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return valid ? m : 0ull;
}

// SCAN: `base` is the histogram itself (E x nchunk, at most kPlaceScanMax
// entries): every block sums it for its chunk's first rows and the experts'
// totals (integer sums, exact in any order), and block 0 writes counts and
// offsets -- the k_scan launch is then not needed.
constexpr int kPlaceScanMax = 16384;
template <bool SCAN>
__global__ __launch_bounds__(256) void k_place(const int32_t *__restrict__ idx, int64_t R, int E,
                                               int chunk, int nchunk, int nbits,
                                               const int32_t *__restrict__ base,
                                               int32_t *__restrict__ slot_to_row,
                                               int32_t *__restrict__ row_to_slot,
                                               int32_t *__restrict__ counts,
                                               int32_t *__restrict__ offsets) {
  __shared__ int cnt[4][kMaxExperts];
  __shared__ int s_base[SCAN ? kMaxExperts : 1], s_tot[SCAN ? kMaxExperts : 1];
  __shared__ int s_part[SCAN ? 256 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < 4 * E; e += 256) cnt[e / E][e % E] = 0;
  if constexpr (SCAN) {
    // thread i: experts [i*epb, (i+1)*epb); their totals and, for this
    // block, the rows of the earlier chunks
    const int epb = (E + 255) / 256;
    const int e_lo = min(E, (int)threadIdx.x * epb), e_hi = min(E, e_lo + epb);
    int mine = 0;
    for (int e = e_lo; e < e_hi; ++e) {
      const int32_t *h = base + (int64_t)e * nchunk;
      int tot = 0, pre = 0;
#pragma unroll 8
      for (int c = 0; c < nchunk; ++c) {
        const int v = h[c];
        tot += v;
        pre += c < (int)blockIdx.x ? v : 0;
      }
      s_base[e] = pre;
      s_tot[e] = tot;
      mine += tot;
    }
    s_part[threadIdx.x] = mine;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {   // inclusive scan of the 256 parts
      const int v = threadIdx.x >= off ? s_part[threadIdx.x - off] : 0;
      __syncthreads();
      s_part[threadIdx.x] += v;
      __syncthreads();
    }
    int run = s_part[threadIdx.x] - mine;   // rows of the experts before e_lo
    for (int e = e_lo; e < e_hi; ++e) {
      s_base[e] += run;
      if (blockIdx.x == 0) {
        offsets[e] = run;
        counts[e] = s_tot[e];
      }
      run += s_tot[e];
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) offsets[E] = s_part[255];
  }
  __syncthreads();
  const int64_t cbeg = (int64_t)blockIdx.x * chunk;
  const int quarter = chunk / 4;   // multiple of 64
  const int64_t wbeg = cbeg + (int64_t)wave * quarter;
  const int64_t wend = min(wbeg + quarter, R);
  const uint64_t lt = (1ull << lane) - 1ull;
  // pass 1: per-wave counts
  for (int64_t s0 = wbeg; s0 < wend; s0 += 64) {
    const int64_t s = s0 + lane;
    int e = (s < wend) ? idx[s] : -1;
    const bool valid = e >= 0 && e < E;
    const uint64_t m = peers_of(e, valid, nbits);
    if (valid && (m & lt) == 0) cnt[wave][e] += __popcll(m);
  }
  __syncthreads();
  // turn counts into per-wave starting offsets inside the chunk
  for (int e = threadIdx.x; e < E; e += 256) {
    int run = 0;
    for (int w = 0; w < 4; ++w) {
      const int c = cnt[w][e];
      cnt[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  // pass 2: ranks and placement
  for (int64_t s0 = wbeg; s0 < wend; s0 += 64) {
    const int64_t s = s0 + lane;
    int e = (s < wend) ? idx[s] : -1;
    const bool valid = e >= 0 && e < E;
    const uint64_t m = peers_of(e, valid, nbits);
    if (s < wend) {
      if (valid) {
        const int before = cnt[wave][e];
        const int rank = __popcll(m & lt);
        const int row = (SCAN ? s_base[e] : base[(int64_t)e * nchunk + blockIdx.x]) + before + rank;
        slot_to_row[s] = row;
        row_to_slot[row] = (int32_t)s;
        if (rank == 0) cnt[wave][e] = before + __popcll(m);
      } else {
        slot_to_row[s] = -1;
      }
    }
  }
}

// ------------------------------------------------------------------ rows
//
// One wave per piece of a token row (kScatterPiece or kRowPiece 16-byte
// chunks), so that many waves have loads in flight.  A
// token row is read once and written to its k rows (forward permute, combine
// bwd), or its k rows are gathered and summed in fp32, j ascending (combine,
// permute bwd).

// 16-byte chunks per lane: 3 for the row copies (two pieces per 2880-wide
// bf16 row; measured 21.1 against 21.8 us for the gpt-oss-20b-like forward
// permute), 2 for the gathered sums (three pieces; 3 and 4 were slower)
constexpr int kScatterNch = 3, kScatterPiece = 64 * kScatterNch;
constexpr int kRowNch = 2, kRowPiece = 64 * kRowNch;

template <typename T>
struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
};

__device__ __forceinline__ void unpack16(const u32x4_t v, float *f, const bf16_t *) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_bits_to_f32(v[i] & 0xffffu);
    f[2 * i + 1] = bf16_bits_to_f32(v[i] >> 16);
  }
}
__device__ __forceinline__ void unpack16(const u32x4_t v, float *f, const float *) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}
__device__ __forceinline__ u32x4_t pack16(const float *f, const bf16_t *) {
  u32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}
__device__ __forceinline__ u32x4_t pack16(const float *f, const float *) {
  u32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
  return v;
}


// src[t] -> dst[slot_to_row[t*k+j]] for j < k (src may be NULL: no rows);
// optional w_dst[row] = w_src[t*k+j].  One wave per (token, 128-chunk piece
// of the row), lane l copying chunks l and l + 64 of the piece to the k rows;
// the piece-0 wave also moves the weights.
template <typename T>
__global__ __launch_bounds__(256) void k_scatter_rows(const T *__restrict__ src,
                                                      const int32_t *__restrict__ slot_to_row,
                                                      const float *__restrict__ w_src, int64_t ntok,
                                                      int d, int k, T *__restrict__ dst,
                                                      float *__restrict__ w_dst) {
  const int nvec = src ? d * (int)sizeof(T) / 16 : 0;
  const int pieces = nvec > 0 ? (nvec + kScatterPiece - 1) / kScatterPiece : 1;
  const int64_t wid = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t t = wid / pieces;
  if (t >= ntok) return;
  const int piece = (int)(wid - t * pieces);
  const int lane = threadIdx.x & 63;
  const int myr = lane < k ? slot_to_row[t * k + lane] : -1;   // k <= 32
  if (w_dst && piece == 0 && lane < k && myr >= 0) w_dst[myr] = w_src[t * k + lane];
  if (!src) return;
  // the row's pieces are made equal (whole 64-chunk columns): 256 chunks
  // split 128 + 128, not 192 + 64
  const int pw = ((nvec + pieces - 1) / pieces + 63) / 64 * 64;
  const int c0 = piece * pw + lane;
  const u32x4_t *s = reinterpret_cast<const u32x4_t *>(src + t * d);
  u32x4_t v[kScatterNch];
  bool ok[kScatterNch];
#pragma unroll
  for (int h = 0; h < kScatterNch; ++h) {
    ok[h] = 64 * h < pw && c0 + 64 * h < nvec;
    v[h] = u32x4_t{0u, 0u, 0u, 0u};
    if (ok[h]) v[h] = s[c0 + 64 * h];
  }
  for (int j = 0; j < k; ++j) {
    const int r = __builtin_amdgcn_readlane(myr, j);
    if (r < 0) continue;
    u32x4_t *o = reinterpret_cast<u32x4_t *>(dst + (int64_t)r * d);
#pragma unroll
    for (int h = 0; h < kScatterNch; ++h)
      if (ok[h]) o[c0 + 64 * h] = v[h];
  }
}

// blocks (4 waves each) of the row kernels for ntok tokens of d elements
template <typename V>
static unsigned row_blocks(int64_t ntok, int d, bool rows = true, int piece = kRowPiece) {
  const int64_t nvec = rows ? (int64_t)d * (int64_t)sizeof(V) / 16 : 0;
  const int64_t pieces = nvec > 0 ? (nvec + piece - 1) / piece : 1;
  return (unsigned)((ntok * pieces + 3) / 4);
}

// The same from the unpermuted dY in token order: each token row is read
// once and its k scaled copies written, S[slot_to_row[t*k+j]] =
// store(w[that row] * dY[t]).  One wave per (token, piece of 192 16-byte
// chunks), three chunks per lane (two pieces per 2880-wide bf16 row).
constexpr int kRsNch = 3, kRsPiece = 64 * kRsNch;
__global__ __launch_bounds__(256) void k_row_scale_scatter(const bf16_t *__restrict__ dy,
                                                           const int32_t *__restrict__ slot_to_row,
                                                           const float *__restrict__ w,
                                                           int64_t ntok, int d, int k,
                                                           bf16_t *__restrict__ s) {
  const int nvec = d / 8;
  const int pieces = (nvec + kRsPiece - 1) / kRsPiece;
  const int64_t wid =
      (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t t = wid / pieces;
  if (t >= ntok) return;
  const int lane = threadIdx.x & 63;
  // equal pieces of whole 64-chunk columns (256 chunks: 128 + 128)
  const int pw = ((nvec + pieces - 1) / pieces + 63) / 64 * 64;
  const int c0 = (int)(wid - t * pieces) * pw + lane;   // chunk h: c0 + 64 h
  const int myr = lane < k ? slot_to_row[t * k + lane] : -1;   // k <= 32
  const float myw = (myr >= 0 && w) ? w[myr] : 1.0f;
  const u32x4_t *src = reinterpret_cast<const u32x4_t *>(dy + t * d);
  u32x4_t x[kRsNch];
  bool ok[kRsNch];
#pragma unroll
  for (int h = 0; h < kRsNch; ++h) {
    ok[h] = 64 * h < pw && c0 + 64 * h < nvec;
    x[h] = u32x4_t{0u, 0u, 0u, 0u};
    if (ok[h]) x[h] = src[c0 + 64 * h];
  }
  for (int j = 0; j < k; ++j) {
    const int r = __builtin_amdgcn_readlane(myr, j);
    if (r < 0) continue;
    const float wr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myw), j));
    u32x4_t *o = reinterpret_cast<u32x4_t *>(s + (int64_t)r * d);
#pragma unroll
    for (int h = 0; h < kRsNch; ++h) {
      u32x4_t y;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        y[q] = pack_bf16x2(bf16_bits_to_f32(x[h][q] & 0xffffu) * wr, bf16_bits_to_f32(x[h][q] >> 16) * wr);
      if (ok[h]) o[c0 + 64 * h] = y;
    }
  }
}

// ---- persistent, software-pipelined row kernels (top-k <= 8)
//
// The one-wave-per-piece kernels above issue a piece's loads, wait for them
// and store: a wave never has two pieces in flight, and the forward permute's
// reads all come before its writes.  These kernels run a grid of a few
// blocks per CU whose waves walk the (token, piece) units u = w, w + W,
// w + 2W, ... and keep two units in flight: the loads of unit n + 1 are
// issued before unit n's sums and stores.  Measured at the gpt-oss-20b-like
// shape (T = 4096, d = 2880, k = 4; kernel durations in a trace): the
// combine 21.1 -> 19.5 us, S = w dY 23.2 -> 21.0 us, the forward permute
// unchanged (19.5 -> 19.4 us).  Larger inputs keep the one-wave kernels
// (row_persist_ok).
//
// Every access is issued unconditionally through a buffer resource; a
// masked one (past the row, a dropped slot, j >= k, a unit past the end)
// takes an offset past the resource, where loads read zero and stores are
// dropped.  The per-unit count of memory operations is then fixed, so the
// wait before unit n's stores leaves unit n + 1's loads and unit n - 1's
// stores in flight; with stores under branches the compiler has to assume
// none were issued and waits for them all.  In-range offsets are below
// kDrop, which the host checks (byte extents below 2^31).
constexpr uint32_t kDrop = 0x80000000u;
constexpr int kRowGridPerCu = 4;   // blocks of 4 waves per CU (3-8 measured alike)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void *base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)(uint32_t)bytes,
                                           0x00020000);
}
// volatile (bit 31 of the cache-policy operand): keeps each load where it is
// written, ahead of the previous unit's sums and stores
__device__ __forceinline__ u32x4_t row_load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(u32x4_t,
                            __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, (int)kDrop));
}

// (token, piece) cursor of a wave's unit sequence, advanced by the W waves
// of the grid without a division per unit
struct RowCur {
  int t, p;
};
struct RowWalk {
  int pieces, dq, dr;
  __device__ RowWalk(int pieces_, int nw) : pieces(pieces_), dq(nw / pieces_), dr(nw % pieces_) {}
  __device__ RowCur first(int w) const { return RowCur{w / pieces, w % pieces}; }
  __device__ RowCur next(RowCur c) const {
    c.p += dr;
    c.t += dq;
    if (c.p >= pieces) {
      c.p -= pieces;
      ++c.t;
    }
    return c;
  }
};

// dst[slot_to_row[t*k+j]] = src[t] for j < k <= KMAX, as k_scatter_rows;
// a piece is three 16-byte chunks per lane.  MODE kRowCopy: rows only;
// kRowCopyW: also w_dst[that row] = w[t*k+j] (w by slot); kRowScale (bf16):
// the copies scaled, store(w[that row] * src[t]) as k_row_scale_scatter (w
// by row: a load behind the slot index, issued when the unit's stores are
// next, which then wait for the previous unit's stores).
constexpr int kRowCopy = 0, kRowCopyW = 1, kRowScale = 2;
template <typename T, int MODE, int KMAX>
__global__ __launch_bounds__(256) void k_scatter_rows_persist(
    const T *__restrict__ src, const int32_t *__restrict__ slot_to_row,
    const float *__restrict__ w, int ntok, int d, int k, T *__restrict__ dst,
    uint64_t dst_bytes, float *__restrict__ w_dst) {
  constexpr bool WS = MODE == kRowCopyW, SC = MODE == kRowScale;
  static_assert(!SC || sizeof(T) == 2, "scaled rows are bf16");
  constexpr int NCH = kScatterNch;
  const int nvec = d * (int)sizeof(T) / 16;
  const int pieces = (nvec + 64 * NCH - 1) / (64 * NCH);
  const int pw = ((nvec + pieces - 1) / pieces + 63) / 64 * 64;   // equal pieces
  const RowWalk walk(pieces, (int)gridDim.x * 4);
  const int lane = threadIdx.x & 63;
  const int lk = lane < k ? lane : k - 1;
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(src, (uint64_t)ntok * nvec * 16);
  const __amdgpu_buffer_rsrc_t rd = row_rsrc(dst, dst_bytes);
  const __amdgpu_buffer_rsrc_t rw = row_rsrc(w_dst, WS ? (uint64_t)ntok * k * 4 : 0);
  // slot indices (and weights) of a unit's token, from a clamped address;
  // lane j >= k holds lane k-1's entry, never read as a row
  auto get_idx = [&](RowCur c) {
    return slot_to_row[(int64_t)(c.t < ntok ? c.t : ntok - 1) * k + lk];
  };
  auto get_w = [&](RowCur c) {
    return WS ? w[(int64_t)(c.t < ntok ? c.t : ntok - 1) * k + lk] : 0.0f;
  };
  auto get_wrow = [&](int myr) { return w[myr >= 0 ? myr : 0]; };
  auto load = [&](RowCur c, u32x4_t (&v)[NCH]) {
    const int cc = c.p * pw + lane;
#pragma unroll
    for (int h = 0; h < NCH; ++h) {
      const int col = cc + 64 * h;
      const bool ok = (c.t < ntok) & (64 * h < pw) & (col < nvec);
      v[h] = row_load(rs, ok ? ((uint32_t)c.t * (uint32_t)nvec + (uint32_t)col) * 16u : kDrop);
    }
  };
  auto store = [&](RowCur c, int myr, float wv, const u32x4_t (&v)[NCH]) {
    const bool tv = c.t < ntok;
    const int cc = c.p * pw + lane;
    if (WS) {
      const bool ok = tv & (c.p == 0) & (lane < k) & (myr >= 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(wv), rw,
                                            (int)(ok ? (uint32_t)myr * 4u : kDrop), 0, 0);
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int r = j < k ? __builtin_amdgcn_readlane(myr, j) : -1;
#pragma unroll
      for (int h = 0; h < NCH; ++h) {
        const int col = cc + 64 * h;
        const bool ok = tv & (r >= 0) & (64 * h < pw) & (col < nvec);
        // dropped stores get distinct offsets, so none is merged away
        const uint32_t off = ok ? ((uint32_t)r * (uint32_t)nvec + (uint32_t)col) * 16u
                                : kDrop + (uint32_t)(j * NCH + h) * 16u;
        u32x4_t y = v[h];
        if (SC) {
          const float wr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), j));
#pragma unroll
          for (int q = 0; q < 4; ++q)
            y[q] = pack_bf16x2(bf16_bits_to_f32(v[h][q] & 0xffffu) * wr,
                               bf16_bits_to_f32(v[h][q] >> 16) * wr);
        }
        __builtin_amdgcn_raw_buffer_store_b128(y, rd, (int)off, 0, 0);
      }
    }
  };
  RowCur ca = walk.first((int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)));
  int ia = get_idx(ca);
  float wa = get_w(ca);
  u32x4_t va[NCH], vb[NCH];
  load(ca, va);
  __builtin_amdgcn_sched_barrier(0);
  {   // dropped stores, as many as a unit issues: the loop is then entered
      // with the same operations behind unit ca's loads on every path
    const u32x4_t z[NCH] = {};
    store(RowCur{ntok, 0}, -1, 0.0f, z);
  }
  do {   // a wave without a unit runs once, every access dropped
    const RowCur cb = walk.next(ca);
    if (SC) wa = get_wrow(ia);
    const int ib = get_idx(cb);
    float wb = get_w(cb);
    load(cb, vb);
    __builtin_amdgcn_sched_barrier(0);
    store(ca, ia, wa, va);
    ca = walk.next(cb);
    if (SC) wb = get_wrow(ib);
    ia = get_idx(ca);
    wa = get_w(ca);
    load(ca, va);
    __builtin_amdgcn_sched_barrier(0);
    store(cb, ib, wb, vb);
  } while (ca.t < ntok);
}

// dst[t] = store(sum_j src[slot_to_row[t*k+j]]), j ascending in fp32, for
// k <= KMAX, as k_gather_sum without the add and router terms.  A unit loads
// KMAX rows of NCH 16-byte chunks per lane.
template <typename T, int KMAX, int NCH>
__global__ __launch_bounds__(256) void k_gather_sum_persist(const T *__restrict__ src,
                                                            uint64_t src_bytes,
                                                            const int32_t *__restrict__ slot_to_row,
                                                            int ntok, int d, int k,
                                                            T *__restrict__ dst) {
  constexpr int N = Vec16<T>::N;
  const int nvec = d * (int)sizeof(T) / 16;
  const int pieces = (nvec + 64 * NCH - 1) / (64 * NCH);
  const RowWalk walk(pieces, (int)gridDim.x * 4);
  const int lane = threadIdx.x & 63;
  const int lk = lane < k ? lane : k - 1;
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(src, src_bytes);
  const __amdgpu_buffer_rsrc_t rd = row_rsrc(dst, (uint64_t)ntok * nvec * 16);
  auto get_idx = [&](RowCur c) {
    return slot_to_row[(int64_t)(c.t < ntok ? c.t : ntok - 1) * k + lk];
  };
  // row of slot j of unit c (-1: none); myr was loaded one half earlier
  auto row_of = [&](RowCur c, int myr, int j) {
    return (j < k) & (c.t < ntok) ? __builtin_amdgcn_readlane(myr, j) : -1;
  };
  auto load = [&](RowCur c, int myr, u32x4_t (&v)[KMAX][NCH]) {
    const int cc = c.p * 64 * NCH + lane;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int r = row_of(c, myr, j);
#pragma unroll
      for (int h = 0; h < NCH; ++h) {
        const int col = cc + 64 * h;
        const bool ok = (r >= 0) & (col < nvec);
        v[j][h] = row_load(rs, ok ? ((uint32_t)r * (uint32_t)nvec + (uint32_t)col) * 16u : kDrop);
      }
    }
  };
  auto sum_store = [&](RowCur c, int myr, const u32x4_t (&v)[KMAX][NCH]) {
    const int cc = c.p * 64 * NCH + lane;
    float acc[NCH][N];
#pragma unroll
    for (int h = 0; h < NCH; ++h)
#pragma unroll
      for (int i = 0; i < N; ++i) acc[h][i] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (row_of(c, myr, j) < 0) continue;
#pragma unroll
      for (int h = 0; h < NCH; ++h) {
        float f[N];
        unpack16(v[j][h], f, (const T *)nullptr);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[h][i] += f[i];
      }
    }
#pragma unroll
    for (int h = 0; h < NCH; ++h) {
      const int col = cc + 64 * h;
      const bool ok = (c.t < ntok) & (col < nvec);
      const uint32_t off = ok ? ((uint32_t)c.t * (uint32_t)nvec + (uint32_t)col) * 16u
                              : kDrop + (uint32_t)h * 16u;
      __builtin_amdgcn_raw_buffer_store_b128(pack16(acc[h], (const T *)nullptr), rd, (int)off, 0,
                                             0);
    }
  };
  RowCur ca = walk.first((int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)));
  RowCur cb = walk.next(ca);
  int ia = get_idx(ca), ib = get_idx(cb);
  u32x4_t va[KMAX][NCH], vb[KMAX][NCH];
  load(ca, ia, va);
  do {   // a wave without a unit runs once, every access dropped
    const RowCur cc2 = walk.next(cb), cc3 = walk.next(cc2);
    const int ic = get_idx(cc2);
    load(cb, ib, vb);
    __builtin_amdgcn_sched_barrier(0);
    sum_store(ca, ia, va);
    const int id = get_idx(cc3);
    load(cc2, ic, va);
    __builtin_amdgcn_sched_barrier(0);
    sum_store(cb, ib, vb);
    ca = cc2;
    cb = cc3;
    ia = ic;
    ib = id;
  } while (ca.t < ntok);
}

// dst[t] = store(sum_j src[slot_to_row[t*k+j]] (+ add[t])), j ascending in
// fp32.  With ROUTER the fp32 term added is the router's share of the token
// gradient, d_logits[t,:] . w_r, formed here as an fma chain over the experts
// in ascending order that skips zero entries (the same chain, bit for bit, as
// the router's own dX kernel), so it is never stored.
// One wave per (token, piece of 64 * kRowNch chunks of the row; 64 with the
// router term): lane l covers 16-byte chunks l, l + 64, ... of the piece.  Row indices are held one per lane and
// read out with readlane; four rows' loads (and four router rows' loads) are
// issued before their adds.

template <typename T, bool ROUTER>
__global__ __launch_bounds__(256) void k_gather_sum(const T *__restrict__ src,
                                                    const int32_t *__restrict__ slot_to_row,
                                                    const float *__restrict__ add,
                                                    const float *__restrict__ d_logits,
                                                    const T *__restrict__ w_r, int E, int64_t ntok,
                                                    int d, int k, T *__restrict__ dst) {
  constexpr int N = Vec16<T>::N;
  const int nvec = d * (int)sizeof(T) / 16;
  // the router term needs more registers: one chunk per lane, more waves
  constexpr int NCH = ROUTER ? 1 : kRowNch;
  constexpr int PIECE = 64 * NCH;
  const int pieces = (nvec + PIECE - 1) / PIECE;
  const int64_t wid = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t t = wid / pieces;
  if (t >= ntok) return;
  const int lane = threadIdx.x & 63;
  const int c0 = (int)(wid - t * pieces) * PIECE + lane;   // chunk h of the lane: c0 + 64 h
  const int myr = lane < k ? slot_to_row[t * k + lane] : -1;   // k <= 32
  // router: this lane's entry of the first 64 experts and the nonzero ones
  const float dl0 = ROUTER && lane < E ? d_logits[t * E + lane] : 0.0f;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  bool vh[NCH];
#pragma unroll
  for (int h = 0; h < NCH; ++h) vh[h] = c0 + 64 * h < nvec;
  float acc[NCH][N];
#pragma unroll
  for (int h = 0; h < NCH; ++h)
#pragma unroll
    for (int i = 0; i < N; ++i) acc[h][i] = 0.0f;
  // Up to four router rows (the first nonzero experts) are loaded with the
  // first four gathered rows; their fmas come after the row sums.
  uint64_t nz = ROUTER ? __ballot(dl0 != 0.0f) : 0;
  int ev[4];
  float g[4];
  u32x4_t wv[4][NCH];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    ev[u] = -1;
    g[u] = 0.0f;
#pragma unroll
    for (int h = 0; h < NCH; ++h) wv[u][h] = zero;
  }
  auto load_router = [&](int e0, float dl) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ev[u] = -1;
      if (nz) {
        const int e = __builtin_ctzll(nz);
        nz &= nz - 1;
        ev[u] = e;
        g[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dl), e));
        const u32x4_t *wr = reinterpret_cast<const u32x4_t *>(w_r + (int64_t)(e0 + e) * d);
#pragma unroll
        for (int h = 0; h < NCH; ++h) wv[u][h] = vh[h] ? wr[c0 + 64 * h] : zero;
      }
    }
  };
  if (ROUTER) load_router(0, dl0);
  for (int j = 0; j < k; j += 4) {
    u32x4_t xv[4][NCH];
    int r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      r[u] = j + u < k ? __builtin_amdgcn_readlane(myr, j + u) : -1;
#pragma unroll
      for (int h = 0; h < NCH; ++h) xv[u][h] = zero;
      if (r[u] >= 0) {
        const u32x4_t *row = reinterpret_cast<const u32x4_t *>(src + (int64_t)r[u] * d);
#pragma unroll
        for (int h = 0; h < NCH; ++h)
          if (vh[h]) xv[u][h] = row[c0 + 64 * h];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (r[u] < 0) continue;
#pragma unroll
      for (int h = 0; h < NCH; ++h) {
        float f[N];
        unpack16(xv[u][h], f, (const T *)nullptr);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[h][i] += f[i];
      }
    }
  }
  if (add) {
    const float *ar = add + t * d;
#pragma unroll
    for (int h = 0; h < NCH; ++h) {
      if (!vh[h]) continue;
      const int64_t c = (int64_t)(c0 + 64 * h) * N;
#pragma unroll
      for (int i = 0; i < N; i += 4) {
        const float4 a4 = *reinterpret_cast<const float4 *>(ar + c + i);
        acc[h][i] += a4.x;
        acc[h][i + 1] += a4.y;
        acc[h][i + 2] += a4.z;
        acc[h][i + 3] += a4.w;
      }
    }
  }
  if (ROUTER) {
    float ra[NCH][N];
#pragma unroll
    for (int h = 0; h < NCH; ++h)
#pragma unroll
      for (int i = 0; i < N; ++i) ra[h][i] = 0.0f;
    for (int e0 = 0; e0 < E; e0 += 64) {
      float dl = dl0;
      if (e0 > 0) {
        dl = e0 + lane < E ? d_logits[t * E + e0 + lane] : 0.0f;
        nz = __ballot(dl != 0.0f);
        load_router(e0, dl);
      }
      while (true) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (ev[u] < 0) continue;
#pragma unroll
          for (int h = 0; h < NCH; ++h) {
            float fw[N];
            unpack16(wv[u][h], fw, (const T *)nullptr);
#pragma unroll
            for (int i = 0; i < N; ++i) ra[h][i] = fmaf(g[u], fw[i], ra[h][i]);
          }
        }
        if (!nz) break;
        load_router(e0, dl);
      }
    }
#pragma unroll
    for (int h = 0; h < NCH; ++h)
#pragma unroll
      for (int i = 0; i < N; ++i) acc[h][i] += ra[h][i];
  }
  u32x4_t *o = reinterpret_cast<u32x4_t *>(dst + t * d);
#pragma unroll
  for (int h = 0; h < NCH; ++h)
    if (vh[h]) o[c0 + 64 * h] = pack16(acc[h], (const T *)nullptr);
}


// CUs of the current device (cached per device)
static unsigned device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return (unsigned)cus[dev];
}

// Blocks of the persistent row kernels: kRowGridPerCu per CU, never more
// than the one-wave-per-piece grid would have.
static unsigned row_grid(unsigned blocks) {
  const unsigned g = device_cus() * kRowGridPerCu;
  return blocks < g ? blocks : g;
}

// The persistent kernels take top-k <= 8, keep every in-range byte offset
// (T*k rows of d elements) below kDrop, and pay off only while the
// one-wave-per-piece grid (`units` waves) is at most two rounds of resident
// waves (32 per CU): with more rounds those kernels already overlap one
// wave's reads with another's writes.  Measured, persistent against one wave
// per piece: 4096 tokens (about one round) 21.5 -> 21.0 us (forward permute),
// 23.5 -> 21.4 us (combine); the Qwen3-30B-A3B-like layer (32768 tokens,
// top-8) 211 -> 226 us, 247 -> 253 us; 16384 tokens mixed within +-4%
// (event timing).
static bool row_persist_ok(int64_t T, int d, int k, size_t elem, int64_t units) {
  return T > 0 && k <= 8 && (uint64_t)T * (uint64_t)k * (uint64_t)d * elem < (uint64_t)kDrop &&
         units <= (int64_t)device_cus() * 64;
}

// src[t] -> dst[slot_to_row[t*k+j]] (and w_dst) for T tokens
template <typename T>
static int launch_scatter(const char *name, const T *src, const int32_t *slot_to_row,
                          const float *w_src, int64_t ntok, int d, int k, T *dst, float *w_dst,
                          hipStream_t s) {
  const unsigned blocks = row_blocks<T>(ntok, d, src != nullptr, kScatterPiece);
  if (src && row_persist_ok(ntok, d, k, sizeof(T), 4 * (int64_t)blocks)) {
    const unsigned g = row_grid(blocks);
    const uint64_t db = (uint64_t)ntok * k * d * sizeof(T);
    const int n = (int)ntok;
    if (k <= 4) {
      if (w_dst)
        MOE_LAUNCH(name, s, k_scatter_rows_persist<T, kRowCopyW, 4><<<g, 256, 0, s>>>(
                                src, slot_to_row, w_src, n, d, k, dst, db, w_dst));
      else
        MOE_LAUNCH(name, s, k_scatter_rows_persist<T, kRowCopy, 4><<<g, 256, 0, s>>>(
                                src, slot_to_row, w_src, n, d, k, dst, db, w_dst));
    } else {
      if (w_dst)
        MOE_LAUNCH(name, s, k_scatter_rows_persist<T, kRowCopyW, 8><<<g, 256, 0, s>>>(
                                src, slot_to_row, w_src, n, d, k, dst, db, w_dst));
      else
        MOE_LAUNCH(name, s, k_scatter_rows_persist<T, kRowCopy, 8><<<g, 256, 0, s>>>(
                                src, slot_to_row, w_src, n, d, k, dst, db, w_dst));
    }
  } else {
    MOE_LAUNCH(name, s, k_scatter_rows<T><<<blocks, 256, 0, s>>>(src, slot_to_row, w_src, ntok, d,
                                                                  k, dst, w_dst));
  }
  return check_launch(name);
}

// dst[t] = store(sum_j src[slot_to_row[t*k+j]] (+ add[t])) for T tokens
template <typename T>
static int launch_gather(const char *name, const T *src, const int32_t *slot_to_row,
                         const float *add, int64_t ntok, int d, int k, T *dst, hipStream_t s) {
  const unsigned blocks = row_blocks<T>(ntok, d, true, k <= 4 ? 192 : 64);
  if (!add && row_persist_ok(ntok, d, k, sizeof(T), 4 * (int64_t)blocks)) {
    const uint64_t sb = (uint64_t)ntok * k * d * sizeof(T);
    const int n = (int)ntok;
    if (k <= 4) {
      // three chunks per lane: 21.3-21.4 us at the gpt-oss-20b-like shape,
      // against 21.6-21.9 with two and 22.3 with one
      const unsigned g = row_grid(blocks);
      MOE_LAUNCH(name, s, k_gather_sum_persist<T, 4, 3><<<g, 256, 0, s>>>(src, sb, slot_to_row, n,
                                                                         d, k, dst));
    } else {
      const unsigned g = row_grid(blocks);
      MOE_LAUNCH(name, s, k_gather_sum_persist<T, 8, 1><<<g, 256, 0, s>>>(src, sb, slot_to_row, n,
                                                                         d, k, dst));
    }
  } else {
    MOE_LAUNCH(name, s, k_gather_sum<T, false><<<row_blocks<T>(ntok, d), 256, 0, s>>>(
                            src, slot_to_row, add, nullptr, nullptr, 0, ntok, d, k, dst));
  }
  return check_launch(name);
}

int launch_row_scale_scatter(const bf16_t *dy, const int32_t *slot_to_row, const float *w,
                             int64_t T, int d, int k, bf16_t *s_rows, hipStream_t s) {
  if (T <= 0) return MOE_OK;
  if (!w)   // scaling by one is the copy
    return launch_scatter<bf16_t>("row_scale", dy, slot_to_row, nullptr, T, d, k, s_rows,
                                  nullptr, s);
  const unsigned blocks = row_blocks<bf16_t>(T, d, true, kScatterPiece);
  if (row_persist_ok(T, d, k, sizeof(bf16_t), 4 * (int64_t)blocks)) {
    const unsigned g = row_grid(blocks);
    const uint64_t db = (uint64_t)T * k * d * sizeof(bf16_t);
    if (k <= 4)
      MOE_LAUNCH("row_scale", s, k_scatter_rows_persist<bf16_t, kRowScale, 4><<<g, 256, 0, s>>>(
                                     dy, slot_to_row, w, (int)T, d, k, s_rows, db, nullptr));
    else
      MOE_LAUNCH("row_scale", s, k_scatter_rows_persist<bf16_t, kRowScale, 8><<<g, 256, 0, s>>>(
                                     dy, slot_to_row, w, (int)T, d, k, s_rows, db, nullptr));
  } else {
    const int64_t waves = T * ((d / 8 + kRsPiece - 1) / kRsPiece);
    MOE_LAUNCH("row_scale", s, k_row_scale_scatter<<<(unsigned)((waves + 3) / 4), 256, 0, s>>>(
                                   dy, slot_to_row, w, T, d, k, s_rows));
  }
  return check_launch("row_scale");
}

}  // namespace moe

using namespace moe;

// ====================================================================== C ABI

static int check_rows(const char *fn, int dtype, int64_t T, int d, int k) {
  MOE_REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "%s: T < 0", fn);
  MOE_REQUIRE(dtype == MOE_BF16 || dtype == MOE_F32, MOE_ERR_UNSUPPORTED, "%s: dtype %d", fn,
              dtype);
  MOE_REQUIRE(d > 0 && d % 8 == 0, MOE_ERR_UNSUPPORTED, "%s: d=%d not a positive multiple of 8",
              fn, d);
  MOE_REQUIRE(k >= 1 && k <= kMaxTopK, MOE_ERR_UNSUPPORTED, "%s: k=%d", fn, k);
  MOE_REQUIRE(T * (int64_t)k < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED, "%s: T*k >= 2^31", fn);
  return MOE_OK;
}

extern "C" size_t moe_permute_workspace_size(int64_t T, int E, int k) {
  if (T < 0 || E < 1 || k < 1) return 0;
  PermPlan p = perm_plan(T, E, k);
  const size_t n = (size_t)E * (size_t)p.nchunk;
  return align_up(2 * n * sizeof(int32_t), 256);
}

extern "C" int moe_permute(const void *x, const int32_t *topk_idx, const float *topk_w, int dtype,
                           int64_t T, int d, int E, int k, int32_t *counts, int32_t *offsets,
                           int32_t *slot_to_row, int32_t *row_to_slot, void *x_perm,
                           float *w_perm, void *ws, size_t ws_bytes, void *stream) {
  clear_error();
  int rc = check_rows("moe_permute", dtype, T, d, k);
  if (rc) return rc;
  MOE_REQUIRE(E >= 1 && E <= kMaxExperts && k <= E, MOE_ERR_UNSUPPORTED, "moe_permute: E=%d k=%d",
              E, k);
  MOE_REQUIRE(counts && offsets, MOE_ERR_INVALID_ARG, "moe_permute: null counts/offsets");
  const size_t need = moe_permute_workspace_size(T, E, k);
  MOE_REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE, "moe_permute: workspace %zu < %zu",
              ws_bytes, need);
  if (T > 0) {
    MOE_REQUIRE(topk_idx && slot_to_row && row_to_slot, MOE_ERR_INVALID_ARG,
                "moe_permute: null map pointer");
    MOE_REQUIRE(!x || (x_perm && aligned16(x) && aligned16(x_perm)), MOE_ERR_INVALID_ARG,
                "moe_permute: x / x_perm");
    MOE_REQUIRE(!w_perm || topk_w, MOE_ERR_INVALID_ARG, "moe_permute: w_perm needs topk_w");
  }
  hipStream_t s = (hipStream_t)stream;
  PermPlan p = perm_plan(T, E, k);
  int32_t *hist = (int32_t *)ws;
  int32_t *base = hist + (size_t)E * p.nchunk;
  if (T == 0) {
    // zero counts and offsets with the scan kernel over an all-zero histogram
    MOE_LAUNCH("permute_hist", s,
               k_hist<<<p.nchunk, 256, 0, s>>>(topk_idx, 0, E, p.chunk, p.nchunk, hist));
    MOE_LAUNCH("permute_scan", s,
               k_scan<<<1, 1024, 0, s>>>(hist, E, p.nchunk, base, counts, offsets));
    return check_launch("moe_permute");
  }
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  MOE_LAUNCH("permute_hist", s,
             k_hist<<<p.nchunk, 256, 0, s>>>(topk_idx, p.R, E, p.chunk, p.nchunk, hist));
  if ((int64_t)E * p.nchunk <= kPlaceScanMax) {   // the blocks scan the histogram themselves
    MOE_LAUNCH("permute_place", s,
               k_place<true><<<p.nchunk, 256, 0, s>>>(topk_idx, p.R, E, p.chunk, p.nchunk, nbits,
                                                      hist, slot_to_row, row_to_slot, counts,
                                                      offsets));
  } else {
    MOE_LAUNCH("permute_scan", s,
               k_scan<<<1, 1024, 0, s>>>(hist, E, p.nchunk, base, counts, offsets));
    MOE_LAUNCH("permute_place", s,
               k_place<false><<<p.nchunk, 256, 0, s>>>(topk_idx, p.R, E, p.chunk, p.nchunk, nbits,
                                                       base, slot_to_row, row_to_slot, nullptr,
                                                       nullptr));
  }
  rc = check_launch("moe_permute(maps)");
  if (rc) return rc;
  if (x || w_perm) {
    if (dtype == MOE_BF16)
      rc = launch_scatter<bf16_t>("permute_rows", (const bf16_t *)x, slot_to_row, topk_w, T, d, k,
                                  (bf16_t *)x_perm, w_perm, s);
    else
      rc = launch_scatter<float>("permute_rows", (const float *)x, slot_to_row, topk_w, T, d, k,
                                 (float *)x_perm, w_perm, s);
  }
  return rc;
}

extern "C" int moe_combine(const void *y_perm, const int32_t *slot_to_row, int dtype, int64_t T,
                           int d, int k, void *y, void *stream) {
  clear_error();
  int rc = check_rows("moe_combine", dtype, T, d, k);
  if (rc) return rc;
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(y_perm && slot_to_row && y && aligned16(y_perm) && aligned16(y), MOE_ERR_INVALID_ARG,
              "moe_combine: null or misaligned pointer");
  hipStream_t s = (hipStream_t)stream;
  if (dtype == MOE_BF16)
    return launch_gather<bf16_t>("combine", (const bf16_t *)y_perm, slot_to_row, nullptr, T, d, k,
                                 (bf16_t *)y, s);
  return launch_gather<float>("combine", (const float *)y_perm, slot_to_row, nullptr, T, d, k,
                              (float *)y, s);
}

extern "C" int moe_combine_bwd(const void *dy, const int32_t *slot_to_row, int dtype, int64_t T,
                               int d, int k, void *dy_perm, void *stream) {
  clear_error();
  int rc = check_rows("moe_combine_bwd", dtype, T, d, k);
  if (rc) return rc;
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(dy && slot_to_row && dy_perm && aligned16(dy) && aligned16(dy_perm),
              MOE_ERR_INVALID_ARG, "moe_combine_bwd: null or misaligned pointer");
  hipStream_t s = (hipStream_t)stream;
  if (dtype == MOE_BF16)
    return launch_scatter<bf16_t>("combine_bwd", (const bf16_t *)dy, slot_to_row, nullptr, T, d, k,
                                  (bf16_t *)dy_perm, nullptr, s);
  return launch_scatter<float>("combine_bwd", (const float *)dy, slot_to_row, nullptr, T, d, k,
                               (float *)dy_perm, nullptr, s);
}

extern "C" int moe_permute_bwd(const void *dx_perm, const int32_t *slot_to_row, const float *dx_add,
                               int dtype, int64_t T, int d, int k, void *dx, void *stream) {
  clear_error();
  int rc = check_rows("moe_permute_bwd", dtype, T, d, k);
  if (rc) return rc;
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(dx_perm && slot_to_row && dx && aligned16(dx_perm) && aligned16(dx) &&
                  (!dx_add || aligned16(dx_add)),
              MOE_ERR_INVALID_ARG, "moe_permute_bwd: null or misaligned pointer");
  hipStream_t s = (hipStream_t)stream;
  if (dtype == MOE_BF16)
    return launch_gather<bf16_t>("permute_bwd", (const bf16_t *)dx_perm, slot_to_row, dx_add, T, d,
                                 k, (bf16_t *)dx, s);
  return launch_gather<float>("permute_bwd", (const float *)dx_perm, slot_to_row, dx_add, T, d, k,
                              (float *)dx, s);
}

extern "C" int moe_permute_bwd_router(const void *dx_perm, const int32_t *slot_to_row,
                                      const float *d_logits, const void *w_r, int dtype, int64_t T,
                                      int d, int E, int k, void *dx, void *stream) {
  clear_error();
  int rc = check_rows("moe_permute_bwd_router", dtype, T, d, k);
  if (rc) return rc;
  MOE_REQUIRE(E >= 1 && E <= kMaxExperts, MOE_ERR_UNSUPPORTED, "moe_permute_bwd_router: E=%d", E);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(dx_perm && slot_to_row && d_logits && w_r && dx && aligned16(dx_perm) &&
                  aligned16(w_r) && aligned16(dx),
              MOE_ERR_INVALID_ARG, "moe_permute_bwd_router: null or misaligned pointer");
  hipStream_t s = (hipStream_t)stream;
  const unsigned blocks = dtype == MOE_BF16 ? row_blocks<bf16_t>(T, d, true, 64)
                                            : row_blocks<float>(T, d, true, 64);
  if (dtype == MOE_BF16)
    MOE_LAUNCH("permute_bwd", s,
               k_gather_sum<bf16_t, true><<<blocks, 256, 0, s>>>(
                   (const bf16_t *)dx_perm, slot_to_row, nullptr, d_logits, (const bf16_t *)w_r,
                   E, T, d, k, (bf16_t *)dx));
  else
    MOE_LAUNCH("permute_bwd", s,
               k_gather_sum<float, true><<<blocks, 256, 0, s>>>(
                   (const float *)dx_perm, slot_to_row, nullptr, d_logits, (const float *)w_r, E,
                   T, d, k, (float *)dx));
  return check_launch("moe_permute_bwd_router");
}
