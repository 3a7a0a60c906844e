// A4: pre-eviction top-k per row [IM 2.A, pre-eviction: the retained entries are chosen
// from the indexer's scores before the full prefill].
//
// One block of 1024 threads per row.  Scores become order-preserving 32-bit keys (NaN as
// -inf, -0 as +0).  The select finds the key T of the n_top-th largest candidate and how
// many keys equal to T must be taken: a min/max pass bounds the candidates' keys to
// [lo, lo + 2^w), then each histogram pass splits the current interval into up to 4096
// equal bins (the top 12 bits of key - lo) and keeps the bin holding the n_top-th largest,
// until the interval is one key wide.  Binning relative to the keys' actual range spreads
// them evenly over the bins whatever the scores' magnitude, so the LDS histogram atomics
// rarely collide, and scores within a few binades need only two passes.
// The final pass walks positions in order, 1024 per wave, with ballots for the in-wave
// ranks and one block-wide exchange of wave totals per decision, so loads and stores are
// coalesced.  Among keys equal to T the lowest positions are kept.  Everything is integer
// work, so the result is exact and deterministic.
#include "common.hpp"

namespace kvm {

static constexpr int kTopkThreads = 1024;
static constexpr int kTopkWaves = kTopkThreads / 64;
static constexpr int kTopkRun = 16;   // keys per thread per batch

__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// integer sum over the wave (every lane ends with the total)
__device__ __forceinline__ int group_sum_i(int x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

// Block-wide exclusive prefix of one int per wave (wave order); lane values are the
// wave's total.  Returns the prefix and writes the block total to *total.
__device__ __forceinline__ int wave_prefix(int wave_total, int* s_w, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_w[wave] = wave_total;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int c = s_w[w];
    base += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ I, int32_t* __restrict__ idx,
                                                           int32_t* __restrict__ slot_map, int L, int n_cand,
                                                           int n_top, int keep) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* Ir = I + (size_t)row * L;
  int32_t* sm = slot_map + (size_t)row * L;
  int32_t* ix = idx + (size_t)row * keep;
  __shared__ int s_hist[4096];
  __shared__ int s_w[kTopkWaves];
  __shared__ uint32_t s_mm[2 * kTopkWaves];
  __shared__ uint32_t s_sel[2];  // bin, remaining k

  uint32_t T = 0;
  int k = n_top;
  if (n_top > 0 && n_top < n_cand) {
    // key range of the candidates
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    for (int b0 = 0; b0 < n_cand; b0 += kTopkThreads * kTopkRun) {
      float v[kTopkRun];
#pragma unroll
      for (int j = 0; j < kTopkRun; ++j) {
        const int t = b0 + j * kTopkThreads + tid;
        v[j] = t < n_cand ? Ir[t] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kTopkRun; ++j)
        if (b0 + j * kTopkThreads + tid < n_cand) {
          const uint32_t key = order_key(v[j]);
          kmin = min(kmin, key);
          kmax = max(kmax, key);
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
    }
    if (lane == 0) { s_mm[wave] = kmin; s_mm[kTopkWaves + wave] = kmax; }
    __syncthreads();
    kmin = s_mm[0];
    kmax = s_mm[kTopkWaves];
#pragma unroll
    for (int w = 1; w < kTopkWaves; ++w) { kmin = min(kmin, s_mm[w]); kmax = max(kmax, s_mm[kTopkWaves + w]); }
    __syncthreads();
    // current interval [lo, lo + 2^width) holds every key still in play
    uint32_t lo = kmin;
    const uint32_t span = kmax - kmin;
    int width = span ? 32 - __clz(span) : 0;
    while (width > 0) {
      const int dbits = width < 12 ? width : 12;
      const int shift = width - dbits, nb = 1 << dbits;
      for (int i = tid; i < nb; i += kTopkThreads) s_hist[i] = 0;
      __syncthreads();
      for (int b0 = 0; b0 < n_cand; b0 += kTopkThreads * kTopkRun) {
        float v[kTopkRun];
#pragma unroll
        for (int j = 0; j < kTopkRun; ++j) {
          const int t = b0 + j * kTopkThreads + tid;
          v[j] = t < n_cand ? Ir[t] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kTopkRun; ++j) {
          const uint32_t rel = order_key(v[j]) - lo;   // wraps below lo: out of range
          if (b0 + j * kTopkThreads + tid < n_cand && ((uint64_t)rel >> width) == 0)
            atomicAdd(&s_hist[rel >> shift], 1);
        }
      }
      __syncthreads();
      // thread i owns the bins nb-1-4i .. nb-4-4i (descending); scan their counts
      int c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int bin = nb - 1 - 4 * tid - j;
        c[j] = bin >= 0 ? s_hist[bin] : 0;
        sum += c[j];
      }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      int tot;
      const int excl = wave_prefix(__shfl(incl, 63), s_w, &tot) + incl - sum;
      if (excl < k && excl + sum >= k) {
        int run = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (run + c[j] >= k) {
            s_sel[0] = (uint32_t)(nb - 1 - 4 * tid - j);
            s_sel[1] = (uint32_t)(k - run);
            break;
          }
          run += c[j];
        }
      }
      __syncthreads();
      lo += s_sel[0] << shift;
      k = (int)s_sel[1];
      width = shift;
      __syncthreads();
    }
    T = lo;
  }
  // Final pass: chunks of 1024 x kTopkRun positions; wave w takes 1024 consecutive
  // positions of a chunk, element (j, lane) at w*1024 + 64 j + lane.
  const bool all = n_top >= n_cand;
  const uint64_t below = lanes_below();
  int eq_before = 0, kept_before = 0;
  for (int base = 0; base < L; base += kTopkThreads * kTopkRun) {
    const int p0 = base + wave * 64 * kTopkRun;
    float v[kTopkRun];
#pragma unroll
    for (int j = 0; j < kTopkRun; ++j) {
      const int t = p0 + 64 * j + lane;
      v[j] = t < n_cand ? Ir[t] : 0.f;
    }
    uint64_t selm[kTopkRun], eqm[kTopkRun];
    int eq_w = 0;
#pragma unroll
    for (int j = 0; j < kTopkRun; ++j) {
      const int t = p0 + 64 * j + lane;
      bool sel = false, eq = false;
      if (t < L) {
        if (t >= n_cand || all) {
          sel = true;
        } else if (n_top > 0) {
          const uint32_t key = order_key(v[j]);
          sel = key > T;
          eq = key == T;
        }
      }
      selm[j] = __ballot(sel);
      eqm[j] = __ballot(eq);
      eq_w += __popcll(eqm[j]);
    }
    int tot;
    // keys equal to T: the first k of them in position order are kept
    int eq_rank = eq_before + wave_prefix(eq_w, s_w, &tot);
    eq_before += tot;
    int sel_w = 0;
#pragma unroll
    for (int j = 0; j < kTopkRun; ++j) {
      const bool take = ((eqm[j] >> lane) & 1ull) && eq_rank + __popcll(eqm[j] & below) < k;
      eq_rank += __popcll(eqm[j]);
      selm[j] |= __ballot(take);
      sel_w += __popcll(selm[j]);
    }
    int slot0 = kept_before + wave_prefix(sel_w, s_w, &tot);
    kept_before += tot;
#pragma unroll
    for (int j = 0; j < kTopkRun; ++j) {
      const int t = p0 + 64 * j + lane;
      const int slot = slot0 + __popcll(selm[j] & below);
      if (t < L) {
        if ((selm[j] >> lane) & 1ull) {
          sm[t] = slot;
          if (slot < keep) ix[slot] = t;
        } else {
          sm[t] = -(t - slot + 1);
        }
      }
      slot0 += __popcll(selm[j]);
    }
  }
}

// ------------------------------------------------------------------ rows held in registers
// Rows of at most 1024 R positions: every thread loads its R scores once, as keys, and all
// passes work from registers.  Element j of lane l in wave w is position w 64 R + 64 j + l,
// so a wave's positions are contiguous (the layout the final ranking needs).  The two
// histograms alternate (the next pass's buffer is cleared while the current one is
// scanned), so a pass costs three block barriers, and the final ranking takes the counts of
// keys above T and equal to T in one block-wide exchange: the equal keys taken before a wave
// are min(equal keys before it, k).  Same keys, bins and order rule as topk_kernel, so the
// result is the same, bit for bit, with a third of the barriers (measured per 16384-position
// row: ~22 barrier-separated phases of 1-2 us each in topk_kernel).
template <int R>
__global__ __launch_bounds__(kTopkThreads) void topk_reg_kernel(const float* __restrict__ I, int32_t* __restrict__ idx,
                                                              int32_t* __restrict__ slot_map, int L, int n_cand,
                                                              int n_top, int keep) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* sm = slot_map + (size_t)row * L;
  int32_t* ix = idx + (size_t)row * keep;
  __shared__ int s_hist[2][4096];
  __shared__ uint32_t s_mm[2 * kTopkWaves];
  __shared__ int s_wt[2 * kTopkWaves];
  __shared__ uint32_t s_sel[2];

  // scores of the candidates (positions < n_cand); loads past them read zeros
  const __amdgpu_buffer_rsrc_t rI = make_rsrc(I + (size_t)row * L, n_cand * 4);
  const int p0 = wave * 64 * R + lane;
  uint32_t key[R];
#pragma unroll
  for (int j = 0; j < R; ++j)
    key[j] = order_key(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rI, (uint32_t)(p0 + 64 * j) * 4u, 0, 0)));
  const bool all = n_top >= n_cand;
  uint32_t T = 0;
  int k = n_top;
  if (n_top > 0 && !all) {
    for (int i = tid; i < 2 * 4096; i += kTopkThreads) (&s_hist[0][0])[i] = 0;
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (p0 + 64 * j < n_cand) {
        kmin = min(kmin, key[j]);
        kmax = max(kmax, key[j]);
      }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
    }
    if (lane == 0) { s_mm[wave] = kmin; s_mm[kTopkWaves + wave] = kmax; }
    __syncthreads();   // also orders the histogram clear before the first pass
    kmin = s_mm[0];
    kmax = s_mm[kTopkWaves];
#pragma unroll
    for (int w = 1; w < kTopkWaves; ++w) { kmin = min(kmin, s_mm[w]); kmax = max(kmax, s_mm[kTopkWaves + w]); }
    // the interval [lo, lo + 2^width) holds every key still in play
    uint32_t lo = kmin;
    const uint32_t span = kmax - kmin;
    int width = span ? 32 - __clz(span) : 0;
    int buf = 0;
    while (width > 0) {
      const int dbits = width < 12 ? width : 12;
      const int shift = width - dbits, nb = 1 << dbits;
      int* h = s_hist[buf];
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const uint32_t rel = key[j] - lo;   // wraps below lo: out of range
        if (p0 + 64 * j < n_cand && ((uint64_t)rel >> width) == 0) atomicAdd(&h[rel >> shift], 1);
      }
      __syncthreads();
      // thread i owns the bins nb-1-4i .. nb-4-4i (descending); scan their counts
      int c[4], sum = 0;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int bin = nb - 1 - 4 * tid - jj;
        c[jj] = bin >= 0 ? h[bin] : 0;
        sum += c[jj];
      }
      // the other buffer was last read before the previous pass's final barrier: clear it for
      // the next pass
      int* ho = s_hist[buf ^ 1];
      for (int i = tid; i < 4096; i += kTopkThreads) ho[i] = 0;
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      if (lane == 63) s_wt[wave] = incl;
      __syncthreads();
      int excl = incl - sum;
#pragma unroll
      for (int w = 0; w < kTopkWaves; ++w) excl += w < wave ? s_wt[w] : 0;
      if (excl < k && excl + sum >= k) {
        int run = excl;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if (run + c[jj] >= k) {
            s_sel[0] = (uint32_t)(nb - 1 - 4 * tid - jj);
            s_sel[1] = (uint32_t)(k - run);
            break;
          }
          run += c[jj];
        }
      }
      __syncthreads();
      lo += s_sel[0] << shift;
      k = (int)s_sel[1];
      width = shift;
      buf ^= 1;
    }
    T = lo;
  }
  // ranking: selected positions get slots in position order; keys equal to T are taken
  // in position order while fewer than k of them are
  const uint64_t below = lanes_below();
  uint64_t gtm[R], eqm[R];
  int gt_w = 0, eq_w = 0;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int p = p0 + 64 * j;
    bool sel = false, eq = false;
    if (p < L) {
      if (p >= n_cand || all) {
        sel = true;
      } else if (n_top > 0) {
        sel = key[j] > T;
        eq = key[j] == T;
      }
    }
    gtm[j] = __ballot(sel);
    eqm[j] = __ballot(eq);
    gt_w += __popcll(gtm[j]);
    eq_w += __popcll(eqm[j]);
  }
  if (lane == 0) { s_wt[wave] = gt_w; s_wt[kTopkWaves + wave] = eq_w; }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    gt_before += w < wave ? s_wt[w] : 0;
    eq_before += w < wave ? s_wt[kTopkWaves + w] : 0;
  }
  int eq_rank = eq_before;
  int slot0 = gt_before + min(eq_before, max(k, 0));
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const bool take = ((eqm[j] >> lane) & 1ull) && eq_rank + __popcll(eqm[j] & below) < k;
    eq_rank += __popcll(eqm[j]);
    const uint64_t selm = gtm[j] | __ballot(take);
    const int p = p0 + 64 * j;
    const int slot = slot0 + __popcll(selm & below);
    if (p < L) {
      if ((selm >> lane) & 1ull) {
        sm[p] = slot;
        if (slot < keep) ix[slot] = p;
      } else {
        sm[p] = -(p - slot + 1);
      }
    }
    slot0 += __popcll(selm);
  }
}

// ------------------------------------------------------------------ wide rows
// Many blocks per row (a workspace is given): each row is cut into chunks of kWChunk
// positions, one block per (chunk, row), and the select runs as a fixed sequence of
// launches, each kernel boundary making the previous step's global results visible:
//   range   each block's candidate key min/max (and the histograms cleared);
//   level l (1..3) every block recomputes the interval [lo, lo + 2^width) and the rank k
//           left from the range and the histograms of levels < l (a 4096-bin scan), then
//           adds its chunk's histogram of the keys in the interval (top 12 bits of
//           key - lo) into level l's global histogram with integer atomics (exact counts);
//           a block whose interval is already one key wide does nothing;
//   count   each block's number of candidates above T and equal to T (T = lo after the
//           levels: 3 x 12 bits cover any 32-bit span);
//   scatter each block takes the counts of the chunks before it (the equal keys are taken in
//           position order: the first k of them), ranks its own positions with ballots and
//           writes slot_map and idx.
// The result is the single-block kernel's, bit for bit: same keys, same order rule.
static constexpr int kWT = 256;                 // threads per block
static constexpr int kWRun = 16;                // positions per thread
static constexpr int kWChunk = kWT * kWRun;     // positions per block
static constexpr int kWBins = 4096;
static constexpr int kWLevels = 3;

struct WideArgs {
  const float* I;
  int32_t* idx;
  int32_t* sm;
  uint32_t* mm;     // [rows][nchunk][2]   chunk key min, max
  uint32_t* hist;   // [rows][levels][4096]
  uint32_t* cnt;    // [rows][nchunk][2]   keys above T, keys equal to T
  uint32_t* state;  // [rows][levels + 1][4]  (lo, width, k) before each level and after the last
  int L, n_cand, n_top, keep, nchunk;
};

// Block-wide exclusive prefix of one int per wave, for kWT threads.
__device__ __forceinline__ int wide_wave_prefix(int wave_total, int* s_w, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_w[wave] = wave_total;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWT / 64; ++w) {
    const int c = s_w[w];
    base += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base;
}

struct WideState {
  uint32_t lo;
  int width, k;
};

// The interval [lo, lo + 2^width) holding every key still in play and the rank k left
// within it.  A state is recomputed by every block of a row from data the previous launch
// completed (identical in every block), and block 0 of the row records it for the launches
// after.
__device__ WideState wide_initial_state(const WideArgs& a, int row, uint32_t* s_sel) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int c = tid; c < a.nchunk; c += kWT) {
    kmin = min(kmin, a.mm[((size_t)row * a.nchunk + c) * 2]);
    kmax = max(kmax, a.mm[((size_t)row * a.nchunk + c) * 2 + 1]);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  if (lane == 0) { s_sel[2 + (tid >> 6)] = kmin; s_sel[6 + (tid >> 6)] = kmax; }
  __syncthreads();
  kmin = s_sel[2];
  kmax = s_sel[6];
#pragma unroll
  for (int w = 1; w < kWT / 64; ++w) { kmin = min(kmin, s_sel[2 + w]); kmax = max(kmax, s_sel[6 + w]); }
  __syncthreads();
  WideState st;
  st.lo = kmin;
  const uint32_t span = kmax - kmin;
  st.width = span ? 32 - __clz(span) : 0;
  st.k = a.n_top;
  return st;
}

__device__ __forceinline__ WideState wide_load_state(const WideArgs& a, int row, int stage) {
  const uint32_t* p = a.state + ((size_t)row * (kWLevels + 1) + stage) * 4;
  WideState st;
  st.lo = p[0];
  st.width = (int)p[1];
  st.k = (int)p[2];
  return st;
}

__device__ __forceinline__ void wide_store_state(const WideArgs& a, int row, int stage, const WideState& st) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    uint32_t* p = a.state + ((size_t)row * (kWLevels + 1) + stage) * 4;
    p[0] = st.lo;
    p[1] = (uint32_t)st.width;
    p[2] = (uint32_t)st.k;
  }
}

// One level: keep the bin of level `l`'s histogram that holds the k-th largest key.
__device__ WideState wide_step(const WideArgs& a, int row, int l, WideState st, int* s_w, uint32_t* s_sel) {
  if (st.width == 0) return st;
  const int tid = threadIdx.x, lane = tid & 63;
  const int dbits = st.width < 12 ? st.width : 12;
  const int shift = st.width - dbits, nb = 1 << dbits;
  const uint32_t* h = a.hist + ((size_t)row * kWLevels + l) * kWBins;
  // thread i owns the 16 bins nb-1-16i .. nb-16-16i (descending)
  int c[16], sum = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int bin = nb - 1 - 16 * tid - j;
    c[j] = bin >= 0 ? (int)h[bin] : 0;
    sum += c[j];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  int tot;
  const int excl = wide_wave_prefix(__shfl(incl, 63), s_w, &tot) + incl - sum;
  if (excl < st.k && excl + sum >= st.k) {
    int run = excl;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (run + c[j] >= st.k) {
        s_sel[0] = (uint32_t)(nb - 1 - 16 * tid - j);
        s_sel[1] = (uint32_t)(st.k - run);
        break;
      }
      run += c[j];
    }
  }
  __syncthreads();
  st.lo += s_sel[0] << shift;
  st.k = (int)s_sel[1];
  st.width = shift;
  __syncthreads();
  return st;
}

// this block's chunk of candidate scores (positions >= n_cand read as 0 and are not used)
__device__ __forceinline__ void wide_load_chunk(const WideArgs& a, int row, int c, float (&v)[kWRun]) {
  const int p0 = c * kWChunk, tid = threadIdx.x;
  const float* Ir = a.I + (size_t)row * a.L;
#pragma unroll
  for (int j = 0; j < kWRun; ++j) {
    const int t = p0 + j * kWT + tid;
    v[j] = t < a.n_cand ? Ir[t] : 0.f;
  }
}

__global__ __launch_bounds__(kWT) void topk_wide_range_kernel(WideArgs a) {
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int p0 = c * kWChunk;
  const float* Ir = a.I + (size_t)row * a.L;
  __shared__ uint32_t s_mm[2 * (kWT / 64)];
  float v[kWRun];
#pragma unroll
  for (int j = 0; j < kWRun; ++j) {
    const int t = p0 + j * kWT + tid;
    v[j] = t < a.n_cand ? Ir[t] : 0.f;
  }
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < kWRun; ++j)
    if (p0 + j * kWT + tid < a.n_cand) {
      const uint32_t key = order_key(v[j]);
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  if (lane == 0) { s_mm[tid >> 6] = kmin; s_mm[kWT / 64 + (tid >> 6)] = kmax; }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int w = 1; w < kWT / 64; ++w) { kmin = min(kmin, s_mm[w]); kmax = max(kmax, s_mm[kWT / 64 + w]); }
    kmin = min(kmin, s_mm[0]);
    kmax = max(kmax, s_mm[kWT / 64]);
    a.mm[((size_t)row * a.nchunk + c) * 2] = kmin;         // a chunk without candidates: (max, 0),
    a.mm[((size_t)row * a.nchunk + c) * 2 + 1] = kmax;     // neutral for the min and the max
  }
  // clear the row's histograms (the level kernels accumulate into them)
  uint32_t* h = a.hist + (size_t)row * kWLevels * kWBins;
  for (int i = c * kWT + tid; i < kWLevels * kWBins; i += a.nchunk * kWT) h[i] = 0u;
}

__global__ __launch_bounds__(kWT) void topk_wide_level_kernel(WideArgs a, int level) {
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  __shared__ int s_w[kWT / 64];
  __shared__ uint32_t s_sel[2 + 2 * (kWT / 64)];
  __shared__ uint32_t s_hist[kWBins];
  float v[kWRun];
  wide_load_chunk(a, row, c, v);   // in flight while the state is worked out
  WideState st = level == 0 ? wide_initial_state(a, row, s_sel)
                            : wide_step(a, row, level - 1, wide_load_state(a, row, level - 1), s_w, s_sel);
  wide_store_state(a, row, level, st);
  if (st.width == 0) return;   // uniform across the row's blocks
  const int dbits = st.width < 12 ? st.width : 12;
  const int shift = st.width - dbits, nb = 1 << dbits;
  for (int i = tid; i < nb; i += kWT) s_hist[i] = 0u;
  __syncthreads();
  const int p0 = c * kWChunk;
#pragma unroll
  for (int j = 0; j < kWRun; ++j) {
    const uint32_t rel = order_key(v[j]) - st.lo;   // wraps below lo: out of range
    if (p0 + j * kWT + tid < a.n_cand && ((uint64_t)rel >> st.width) == 0) atomicAdd(&s_hist[rel >> shift], 1u);
  }
  __syncthreads();
  uint32_t* h = a.hist + ((size_t)row * kWLevels + level) * kWBins;
  for (int i = tid; i < nb; i += kWT)
    if (s_hist[i]) atomicAdd(&h[i], s_hist[i]);
}

__global__ __launch_bounds__(kWT) void topk_wide_count_kernel(WideArgs a) {
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  __shared__ int s_w[kWT / 64];
  __shared__ uint32_t s_sel[2 + 2 * (kWT / 64)];
  float v[kWRun];
  wide_load_chunk(a, row, c, v);
  const WideState st = wide_step(a, row, kWLevels - 1, wide_load_state(a, row, kWLevels - 1), s_w, s_sel);
  wide_store_state(a, row, kWLevels, st);
  const uint32_t T = st.lo;
  const int p0 = c * kWChunk;
  int gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kWRun; ++j) {
    if (p0 + j * kWT + tid < a.n_cand) {
      const uint32_t key = order_key(v[j]);
      gt += key > T;
      eq += key == T;
    }
  }
  int tot_gt, tot_eq;
  gt = group_sum_i(gt);
  eq = group_sum_i(eq);
  wide_wave_prefix(gt, s_w, &tot_gt);
  wide_wave_prefix(eq, s_w, &tot_eq);
  if (tid == 0) {
    a.cnt[((size_t)row * a.nchunk + c) * 2] = (uint32_t)tot_gt;
    a.cnt[((size_t)row * a.nchunk + c) * 2 + 1] = (uint32_t)tot_eq;
  }
}

// mode: 0 = select through T and k (counts in a.cnt), 1 = keep every position, 2 = keep only
// the positions >= n_cand (no candidate is taken)
__global__ __launch_bounds__(kWT) void topk_wide_scatter_kernel(WideArgs a, int mode) {
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_w[kWT / 64];
  __shared__ uint32_t s_sel[2 + 2 * (kWT / 64)];
  (void)s_sel;
  uint32_t T = 0;
  int k = 0;
  if (mode == 0) {
    const WideState st = wide_load_state(a, row, kWLevels);
    T = st.lo;
    k = st.k;
  }
  const int p0 = c * kWChunk;
  // the chunks before this one: kept positions and keys equal to T, in position order
  int sel_before = 0, eq_before = 0;
  if (mode == 0) {
    for (int cc = 0; cc < c; ++cc) {
      const int gt = (int)a.cnt[((size_t)row * a.nchunk + cc) * 2];
      const int ne = (int)a.cnt[((size_t)row * a.nchunk + cc) * 2 + 1];
      const int taken = min(max(k - eq_before, 0), ne);
      sel_before += gt + taken;
      eq_before += ne;
    }
  } else if (mode == 1) {
    sel_before = p0;
  }
  // positions >= n_cand (the recent window) before this chunk are all kept
  if (mode != 1) sel_before += max(0, min(p0, a.L) - a.n_cand);
  const float* Ir = a.I + (size_t)row * a.L;
  int32_t* sm = a.sm + (size_t)row * a.L;
  int32_t* ix = a.idx + (size_t)row * a.keep;
  // wave w takes positions p0 + w*1024 + 64 j + lane
  const int q0 = p0 + wave * 64 * kWRun;
  float v[kWRun];
#pragma unroll
  for (int j = 0; j < kWRun; ++j) {
    const int t = q0 + 64 * j + lane;
    v[j] = t < a.n_cand ? Ir[t] : 0.f;
  }
  const uint64_t below = lanes_below();
  uint64_t selm[kWRun], eqm[kWRun];
  int eq_w = 0;
#pragma unroll
  for (int j = 0; j < kWRun; ++j) {
    const int t = q0 + 64 * j + lane;
    bool sel = false, eq = false;
    if (t < a.L) {
      if (t >= a.n_cand || mode == 1) {
        sel = true;
      } else if (mode == 0) {
        const uint32_t key = order_key(v[j]);
        sel = key > T;
        eq = key == T;
      }
    }
    selm[j] = __ballot(sel);
    eqm[j] = __ballot(eq);
    eq_w += __popcll(eqm[j]);
  }
  int tot;
  int eq_rank = eq_before + wide_wave_prefix(eq_w, s_w, &tot);
  int sel_w = 0;
#pragma unroll
  for (int j = 0; j < kWRun; ++j) {
    const bool take = ((eqm[j] >> lane) & 1ull) && eq_rank + __popcll(eqm[j] & below) < k;
    eq_rank += __popcll(eqm[j]);
    selm[j] |= __ballot(take);
    sel_w += __popcll(selm[j]);
  }
  int slot0 = sel_before + wide_wave_prefix(sel_w, s_w, &tot);
#pragma unroll
  for (int j = 0; j < kWRun; ++j) {
    const int t = q0 + 64 * j + lane;
    const int slot = slot0 + __popcll(selm[j] & below);
    if (t < a.L) {
      if ((selm[j] >> lane) & 1ull) {
        sm[t] = slot;
        if (slot < a.keep) ix[slot] = t;
      } else {
        sm[t] = -(t - slot + 1);
      }
    }
    slot0 += __popcll(selm[j]);
  }
}

struct WideWs {
  size_t mm, hist, cnt, state, total;
  int nchunk;
};
static WideWs wide_ws(int rows, int L) {
  WideWs w;
  w.nchunk = (L + kWChunk - 1) / kWChunk;
  w.mm = 0;
  w.hist = align_up((size_t)rows * w.nchunk * 2 * sizeof(uint32_t), 256);
  w.cnt = align_up(w.hist + (size_t)rows * kWLevels * kWBins * sizeof(uint32_t), 256);
  w.state = align_up(w.cnt + (size_t)rows * w.nchunk * 2 * sizeof(uint32_t), 256);
  w.total = align_up(w.state + (size_t)rows * (kWLevels + 1) * 4 * sizeof(uint32_t), 256);
  return w;
}

// Many blocks per row pay off once a row is long enough that one block's passes over it
// dominate: measured (HIP graphs) the six launches take 32-36 us whatever the row length,
// one block per row 21 us at 16384 positions, 37 us at 32768 and 124 us at 131072.
static constexpr int kWideMinL = 32768 + 1;

}  // namespace kvm

using namespace kvm;

static bool topk_sizes(const kvm_topk_desc* d, int* n_cand, int* n_top, int* keep) {
  if (!d || d->rows <= 0 || d->L <= 0 || d->B < 0 || d->R < 0) return false;
  if (d->recent_inclusive && d->B < d->R) return false;
  const int R = d->R < d->L ? d->R : d->L;
  *n_cand = d->L - R;
  *n_top = d->recent_inclusive ? d->B - d->R : d->B;
  *keep = (*n_top >= *n_cand) ? d->L : *n_top + R;
  return true;
}

extern "C" int32_t kvm_topk_keep(const kvm_topk_desc* d) {
  int nc, nt, keep;
  return topk_sizes(d, &nc, &nt, &keep) ? keep : -1;
}

extern "C" size_t kvm_topk_workspace_size(const kvm_topk_desc* d) {
  int nc, nt, keep;
  if (!topk_sizes(d, &nc, &nt, &keep)) return 0;
  return wide_ws(d->rows, d->L).total;
}

extern "C" kvm_status kvm_topk_select(const kvm_topk_desc* d, const float* I, int32_t* idx, int32_t* slot_map,
                                      void* ws, size_t ws_bytes, void* stream) {
  KVM_PTR(d);
  KVM_REQUIRE(d->rows > 0 && d->L > 0, KVM_ERR_SHAPE, "rows and L must be positive");
  KVM_REQUIRE(d->B >= 0 && d->R >= 0, KVM_ERR_RANGE, "B and R must be non-negative");
  KVM_REQUIRE(!d->recent_inclusive || d->B >= d->R, KVM_ERR_RANGE, "budget %d below recent window %d", d->B, d->R);
  KVM_PTR_ALIGNED(I); KVM_PTR_ALIGNED(idx); KVM_PTR_ALIGNED(slot_map);
  int n_cand, n_top, keep;
  topk_sizes(d, &n_cand, &n_top, &keep);
  const WideWs w = wide_ws(d->rows, d->L);
  if (ws) {
    KVM_REQUIRE(ws_bytes >= w.total, KVM_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
    KVM_ALIGNED(ws);
  }
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->L <= kTopkThreads * 4) {
    hipLaunchKernelGGL(topk_reg_kernel<4>, dim3(d->rows), dim3(kTopkThreads), 0, s, I, idx, slot_map, d->L, n_cand,
                       n_top, keep);
    return check_hip(hipGetLastError(), "topk_reg_kernel launch");
  }
  if (d->L <= kTopkThreads * 16) {
    hipLaunchKernelGGL(topk_reg_kernel<16>, dim3(d->rows), dim3(kTopkThreads), 0, s, I, idx, slot_map, d->L, n_cand,
                       n_top, keep);
    return check_hip(hipGetLastError(), "topk_reg_kernel launch");
  }
  if (!ws || d->L < kWideMinL) {
    hipLaunchKernelGGL(topk_kernel, dim3(d->rows), dim3(kTopkThreads), 0, s, I, idx, slot_map, d->L, n_cand, n_top,
                       keep);
    return check_hip(hipGetLastError(), "topk_kernel launch");
  }
  char* base = static_cast<char*>(ws);
  WideArgs a{I, idx, slot_map, reinterpret_cast<uint32_t*>(base + w.mm), reinterpret_cast<uint32_t*>(base + w.hist),
             reinterpret_cast<uint32_t*>(base + w.cnt), reinterpret_cast<uint32_t*>(base + w.state), d->L, n_cand,
             n_top, keep, w.nchunk};
  const dim3 grid(w.nchunk, d->rows);
  const int mode = n_top >= n_cand ? 1 : (n_top <= 0 ? 2 : 0);
  if (mode == 0) {
    hipLaunchKernelGGL(topk_wide_range_kernel, grid, dim3(kWT), 0, s, a);
    for (int l = 0; l < kWLevels; ++l) hipLaunchKernelGGL(topk_wide_level_kernel, grid, dim3(kWT), 0, s, a, l);
    hipLaunchKernelGGL(topk_wide_count_kernel, grid, dim3(kWT), 0, s, a);
  }
  hipLaunchKernelGGL(topk_wide_scatter_kernel, grid, dim3(kWT), 0, s, a, mode);
  return check_hip(hipGetLastError(), "top-k launches");
}
