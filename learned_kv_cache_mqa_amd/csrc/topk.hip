// A4: pre-eviction top-k per row [IM 2.A, pre-eviction: the retained entries are chosen
// from the indexer's scores before the full prefill].
//
// One block of 1024 threads per row.  Scores become order-preserving 32-bit keys (NaN as
// -inf, -0 as +0); a most-significant-digit radix select with 8-bit digits and LDS
// histograms finds the key T of the n_top-th largest candidate and how many keys equal
// to T must be taken.  A final pass in position order assigns kept slots and eviction
// ranks with wave ballots and a block-wide prefix count; among keys equal to T the lowest
// positions are kept.  Everything is integer work, so the result is exact and
// deterministic.
#include "common.hpp"

namespace kvm {

static constexpr int kTopkThreads = 1024;
static constexpr int kTopkWaves = kTopkThreads / 64;

// Exclusive prefix count of `flag` over the block in thread order; returns the prefix and
// writes the block total to *total.  Uses s_cnt[kTopkWaves + 1].
__device__ __forceinline__ int block_prefix(bool flag, int* s_cnt, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) s_cnt[wave] = __popcll(m);
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int c = s_cnt[w];
    base += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + below;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ I, int32_t* __restrict__ idx,
                                                           int32_t* __restrict__ slot_map, int L, int n_cand,
                                                           int n_top, int keep) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const float* Ir = I + (size_t)row * L;
  int32_t* sm = slot_map + (size_t)row * L;
  int32_t* ix = idx + (size_t)row * keep;
  __shared__ int s_hist[256];
  __shared__ int s_cnt[kTopkWaves + 1];
  __shared__ uint32_t s_sel[2];  // prefix, remaining k

  uint32_t prefix = 0, mask = 0;
  int k = n_top;
  if (n_top > 0 && n_top < n_cand) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kTopkThreads) s_hist[i] = 0;
      __syncthreads();
      for (int t = tid; t < n_cand; t += kTopkThreads) {
        const uint32_t key = order_key(Ir[t]);
        if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l owns digits 255-4l .. 252-4l (descending)
        int c[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) { c[j] = s_hist[255 - 4 * tid - j]; sum += c[j]; }
        int incl = sum;  // inclusive scan over lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(incl, off);
          if (tid >= off) incl += y;
        }
        const int excl = incl - sum;
        if (excl < k && incl >= k) {
          int run = excl;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (run + c[j] >= k) {
              s_sel[0] = (uint32_t)(255 - 4 * tid - j);
              s_sel[1] = (uint32_t)(k - run);
              break;
            }
            run += c[j];
          }
        }
      }
      __syncthreads();
      prefix |= s_sel[0] << shift;
      mask |= 255u << shift;
      k = (int)s_sel[1];
      __syncthreads();
    }
  }
  // T = prefix; among keys == T take the k lowest positions
  const bool all = n_top >= n_cand;
  int eq_before = 0, kept_before = 0;
  for (int base = 0; base < L; base += kTopkThreads) {
    const int t = base + tid;
    const bool valid = t < L;
    bool cand_eq = false, sel = false;
    if (valid) {
      if (t >= n_cand || all) {
        sel = true;
      } else if (n_top > 0) {
        const uint32_t key = order_key(Ir[t]);
        sel = key > prefix;
        cand_eq = key == prefix;
      }
    }
    int tot;
    const int eq_rank = block_prefix(cand_eq, s_cnt, &tot);
    if (cand_eq && eq_before + eq_rank < k) sel = true;
    eq_before += tot;
    const int slot = kept_before + block_prefix(sel, s_cnt, &tot);
    if (valid) {
      if (sel) {
        sm[t] = slot;
        if (slot < keep) ix[slot] = t;
      } else {
        sm[t] = -(t - slot + 1);
      }
    }
    kept_before += tot;
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
