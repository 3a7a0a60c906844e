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

extern "C" kvm_status kvm_topk_select(const kvm_topk_desc* d, const float* I, int32_t* idx, int32_t* slot_map,
                                      void* stream) {
  KVM_PTR(d);
  KVM_REQUIRE(d->rows > 0 && d->L > 0, KVM_ERR_SHAPE, "rows and L must be positive");
  KVM_REQUIRE(d->B >= 0 && d->R >= 0, KVM_ERR_RANGE, "B and R must be non-negative");
  KVM_REQUIRE(!d->recent_inclusive || d->B >= d->R, KVM_ERR_RANGE, "budget %d below recent window %d", d->B, d->R);
  KVM_PTR_ALIGNED(I); KVM_PTR_ALIGNED(idx); KVM_PTR_ALIGNED(slot_map);
  int n_cand, n_top, keep;
  topk_sizes(d, &n_cand, &n_top, &keep);
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;
  hipLaunchKernelGGL(topk_kernel, dim3(d->rows), dim3(kTopkThreads), 0, static_cast<hipStream_t>(stream), I, idx,
                     slot_map, d->L, n_cand, n_top, keep);
  return check_hip(hipGetLastError(), "topk_kernel launch");
}
