// A5 + A6 / V2: one pass over K, V that compacts the kept rows into the head-major cache
// and folds the evicted rows into the latent memory [IM 2.B: decayed outer-product
// accumulation into M and b] or into MomentKV's moment sums [MKV 1].
// Cache layout written: Kc [b, H_kv, cap, d] (slot-major), Vc [b, H_kv, d, cap] (dim-major,
// so that decode's P V product reads 8 consecutive slots of a dim as one 16-byte operand).
//
// The memory build is a contraction over evicted tokens:
//   M_g = sum_i w_i v_i u_i^T,  u_i = phi(k_i) (memory) or k_i (moments), w_i = lam^(n-i) or 1.
// bf16 inputs: a block streams a chunk of positions of one (sequence, KV head) in tiles of
// 32 tokens; V^T and U^T tiles are staged in LDS (token pairs packed per dim row) and the
// d x d partial product runs on the matrix cores (v_mfma_f32_32x32x16_bf16).  V is exact
// in bf16; u = w phi(k) is split into bf16 hi + lo so the product keeps ~16 bits of u.
// fp32 inputs use fp32 FMA.  Partial states per chunk go to the workspace; the last block
// of a (sequence, KV head) sums them in chunk order (deterministic, no float atomics) and
// applies the decay of the previous state: M <- lam^n M + sum_c M_c.
#include "common.hpp"

namespace kvm {

struct CompactArgs {
  const void* K;
  const void* V;
  const int32_t* slot_map;
  void* Kc;
  void* Vc;
  float* M;     // memory: M; moments: S
  float* vec0;  // memory: bvec; moments: s_k
  float* vec1;  // moments: s_v
  int32_t* n_e;
  float* partM;    // [pairs, chunks, D, D]
  float* partv;    // [pairs, chunks, 2, D]
  int* partn;      // [pairs, chunks]
  int* counters;   // [pairs]
  int L, H_kv, cap, n_ev, chunk, n_chunks, per_head;
  long long tok_stride, head_stride, batch_stride;  // elements
  int mode;        // 0 copy, KVM_FUSE_MEM, KVM_FUSE_MOMENTS
  float log2lam;   // log2(lam) (lam > 0)
  double log2lam_d;
  int lam_zero;    // lam == 0
  float lam_n;     // lam^n_ev
};

__device__ __forceinline__ float evict_weight(const CompactArgs& a, int rank) {
  if (a.mode != KVM_FUSE_MEM) return 1.f;
  const int e = a.n_ev - rank;
  if (a.lam_zero) return e == 0 ? 1.f : 0.f;
  return exp2f((float)e * a.log2lam);
}

// ------------------------------------------------------------------ final fixed-order reduce
template <int D>
__device__ void compact_finish(const CompactArgs& a, size_t pair) {
  const int tid = threadIdx.x;
  const float* pm = a.partM + pair * a.n_chunks * (size_t)(D * D);
  const float* pv = a.partv + pair * a.n_chunks * (size_t)(2 * D);
  const bool mem = a.mode == KVM_FUSE_MEM;
  const float dec = mem ? a.lam_n : 1.f;
  float* Mo = a.M + pair * (size_t)(D * D);
  for (int i = tid; i < D * D; i += blockDim.x) {
    float s = 0.f;
    for (int c = 0; c < a.n_chunks; ++c) s += pm[(size_t)c * D * D + i];
    Mo[i] = fmaf(dec, Mo[i], s);
  }
  for (int i = tid; i < 2 * D; i += blockDim.x) {
    if (mem && i >= D) break;
    float s = 0.f;
    for (int c = 0; c < a.n_chunks; ++c) s += pv[(size_t)c * 2 * D + i];
    float* out = (i < D ? a.vec0 : a.vec1) + pair * D;
    const int j = i % D;
    out[j] = fmaf(dec, out[j], s);
  }
  if (!mem && tid == 0) {
    int s = 0;
    for (int c = 0; c < a.n_chunks; ++c) s += a.partn[pair * a.n_chunks + c];
    a.n_e[pair] += s;
  }
}

// ------------------------------------------------------------------ bf16: matrix cores
// LDS tile: per dim row, 16 token pairs (32 tokens, bf16x2 per word) + 2 pad words; a pitch
// of 18 words keeps the transposed stores and the 8-byte fragment loads conflict-light.
constexpr int kTok = 32;
constexpr int kPitch = 18;

template <int D>
__global__ __launch_bounds__(256) void compact_mfma_kernel(CompactArgs a) {
  static_assert(D == 64 || D == 128, "D");
  constexpr int NT = D / 32;               // 32x32 tiles per side
  constexpr int TPW = NT * NT / 4;         // output tiles per wave (4 waves)
  constexpr int DB = D / 8;                // 8-dim blocks per row
  constexpr int PAIRS_PER_PASS = (256 / DB) < (kTok / 2) ? (256 / DB) : (kTok / 2);
  constexpr int PASSES = (kTok / 2) / PAIRS_PER_PASS;
  static_assert(PASSES * PAIRS_PER_PASS == kTok / 2, "tile");
  const int c = blockIdx.x, g = blockIdx.y, bb = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t pair = (size_t)bb * a.H_kv + g;

  __shared__ uint32_t sV[D * kPitch];
  __shared__ uint32_t sH[D * kPitch];
  __shared__ uint32_t sL[D * kPitch];
  __shared__ int s_flag, s_n;

  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.K) + bb * a.batch_stride + g * a.head_stride;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(a.V) + bb * a.batch_stride + g * a.head_stride;
  const int32_t* smr = a.slot_map + (a.per_head ? pair : (size_t)bb) * a.L;
  uint16_t* Kcb = a.Kc ? reinterpret_cast<uint16_t*>(a.Kc) + pair * a.cap * D : nullptr;
  uint16_t* Vcb = a.Vc ? reinterpret_cast<uint16_t*>(a.Vc) + pair * a.cap * D : nullptr;
  const bool fuse = a.mode != 0;

  // thread -> (token pair within pass, 8-dim block)
  const int tp = tid % PAIRS_PER_PASS;
  const int db = tid / PAIRS_PER_PASS;
  const bool loader = db < DB;   // D = 64 leaves half the threads without a load slot
  float vacc0[8], vacc1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { vacc0[e] = 0.f; vacc1[e] = 0.f; }
  int nloc = 0;

  f32x16_t acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[t][j] = 0.f;

  const int p0 = c * a.chunk, p1 = min(a.L, p0 + a.chunk);
  for (int base = p0; base < p1; base += kTok) {
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int pr = ps * PAIRS_PER_PASS + tp;  // pair index in tile
      uint32_t vw[8], hw[8], lw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { vw[e] = 0; hw[e] = 0; lw[e] = 0; }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int t = base + 2 * pr + half;
        if (loader && t < p1) {
          const int s = smr[t];
          const uint4 kr = *reinterpret_cast<const uint4*>(Kb + t * a.tok_stride + db * 8);
          const uint4 vr = *reinterpret_cast<const uint4*>(Vb + t * a.tok_stride + db * 8);
          if (s >= 0) {
            if (Kcb) *reinterpret_cast<uint4*>(Kcb + (size_t)s * D + db * 8) = kr;
            if (Vcb) {   // dim-major V cache
              const uint32_t vv[4] = {vr.x, vr.y, vr.z, vr.w};
#pragma unroll
              for (int e = 0; e < 8; ++e)
                Vcb[(size_t)(db * 8 + e) * a.cap + s] = (uint16_t)((e & 1) ? (vv[e >> 1] >> 16) : (vv[e >> 1] & 0xffffu));
            }
          } else if (fuse) {
            const float w = evict_weight(a, -s);
            float kf[8], vf[8];
            Vec16<uint16_t>::unpack(kr, kf);
            Vec16<uint16_t>::unpack(vr, vf);
            const uint32_t vv[4] = {vr.x, vr.y, vr.z, vr.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float u = a.mode == KVM_FUSE_MEM ? w * phi_f(kf[e]) : kf[e];
              const uint32_t hb = f32_to_bf16_bits(u);
              const uint32_t lb = f32_to_bf16_bits(u - __uint_as_float(hb << 16));
              const uint32_t vb = (e & 1) ? (vv[e >> 1] >> 16) : (vv[e >> 1] & 0xffffu);
              vw[e] |= vb << (16 * half);
              hw[e] |= hb << (16 * half);
              lw[e] |= lb << (16 * half);
              vacc0[e] += u;
              vacc1[e] += vf[e];
            }
            if (db == 0) ++nloc;
          }
        }
      }
      if (fuse && loader) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int row = db * 8 + e;
          sV[row * kPitch + pr] = vw[e];
          sH[row * kPitch + pr] = hw[e];
          sL[row * kPitch + pr] = lw[e];
        }
      }
    }
    if (!fuse) continue;
    __syncthreads();
    // 2 k-steps of 16 tokens; lane (m = lane % 32, kg = lane / 32) reads 8 tokens = 4 words
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int woff = ks * 8 + (lane >> 5) * 4;
      const int m = lane & 31;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int tile = wave * TPW + t;
        const int ti = tile / NT, tj = tile % NT;   // dv tile, dk tile
        const uint32_t* pa = sV + (ti * 32 + m) * kPitch + woff;
        const uint32_t* ph = sH + (tj * 32 + m) * kPitch + woff;
        const uint32_t* pl = sL + (tj * 32 + m) * kPitch + woff;
        const uint2 a0 = *reinterpret_cast<const uint2*>(pa), a1 = *reinterpret_cast<const uint2*>(pa + 2);
        const uint2 h0 = *reinterpret_cast<const uint2*>(ph), h1 = *reinterpret_cast<const uint2*>(ph + 2);
        const uint2 l0 = *reinterpret_cast<const uint2*>(pl), l1 = *reinterpret_cast<const uint2*>(pl + 2);
        const uint4 av = {a0.x, a0.y, a1.x, a1.y}, hv = {h0.x, h0.y, h1.x, h1.y}, lv = {l0.x, l0.y, l1.x, l1.y};
        bf16x8_t A, Bh, Bl;
        __builtin_memcpy(&A, &av, 16);
        __builtin_memcpy(&Bh, &hv, 16);
        __builtin_memcpy(&Bl, &lv, 16);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bh, acc[t], 0, 0, 0);
        if (a.mode == KVM_FUSE_MEM) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bl, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  if (!fuse) return;

  // partial state of this chunk -> workspace
  float* pm = a.partM + (pair * a.n_chunks + c) * (size_t)(D * D);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tile = wave * TPW + t;
    const int ti = tile / NT, tj = tile % NT;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = ti * 32 + 8 * (j / 4) + 4 * (lane / 32) + (j % 4);
      const int col = tj * 32 + (lane & 31);
      pm[r * D + col] = acc[t][j];
    }
  }
  // vector sums: threads sharing db reduce over their token pairs
  float* pv = a.partv + (pair * a.n_chunks + c) * (size_t)(2 * D);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x0 = vacc0[e], x1 = vacc1[e];
    x0 = group_sum<PAIRS_PER_PASS>(x0);
    x1 = group_sum<PAIRS_PER_PASS>(x1);
    if (tp == 0 && loader) { pv[db * 8 + e] = x0; pv[D + db * 8 + e] = x1; }
  }
  if (tid == 0) s_n = 0;
  __syncthreads();
  if (db == 0 && nloc) atomicAdd(&s_n, nloc);
  __syncthreads();
  if (tid == 0) a.partn[pair * a.n_chunks + c] = s_n;
  if (!last_block_ticket(a.counters + pair, a.n_chunks, &s_flag)) return;
  compact_finish<D>(a, pair);
}

// ------------------------------------------------------------------ fp32: FMA
// fp32 inputs are the small workloads; the outer products accumulate in fp64 so that the
// fp32 results carry a rounding error of a few ulp regardless of the evicted count.
template <int D>
__global__ __launch_bounds__(256) void compact_f32_kernel(CompactArgs a) {
  constexpr int EPT = D * D / 256;         // M elements per thread
  const int c = blockIdx.x, g = blockIdx.y, bb = blockIdx.z;
  const int tid = threadIdx.x;
  const size_t pair = (size_t)bb * a.H_kv + g;
  __shared__ double sv[kTok][D];
  __shared__ double su[kTok][D];
  __shared__ int s_flag, s_cnt;
  const float* Kb = reinterpret_cast<const float*>(a.K) + bb * a.batch_stride + g * a.head_stride;
  const float* Vb = reinterpret_cast<const float*>(a.V) + bb * a.batch_stride + g * a.head_stride;
  const int32_t* smr = a.slot_map + (a.per_head ? pair : (size_t)bb) * a.L;
  float* Kcb = a.Kc ? reinterpret_cast<float*>(a.Kc) + pair * a.cap * D : nullptr;
  float* Vcb = a.Vc ? reinterpret_cast<float*>(a.Vc) + pair * a.cap * D : nullptr;
  const bool fuse = a.mode != 0;
  double acc[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) acc[i] = 0.0;
  double v0 = 0.0, v1 = 0.0;  // vector sums for dim tid (tid < D)
  int cnt = 0;
  const int p0 = c * a.chunk, p1 = min(a.L, p0 + a.chunk);
  for (int base = p0; base < p1; base += kTok) {
    for (int i = tid; i < kTok * D; i += 256) {
      const int tt = i / D, dd = i % D, t = base + tt;
      double vv = 0.0, u = 0.0;
      if (t < p1) {
        const float kv = Kb[t * a.tok_stride + dd];
        const float vf = Vb[t * a.tok_stride + dd];
        const int s = smr[t];
        if (s >= 0) {
          if (Kcb) Kcb[(size_t)s * D + dd] = kv;
          if (Vcb) Vcb[(size_t)dd * a.cap + s] = vf;
        } else if (fuse) {
          vv = vf;
          if (a.mode == KVM_FUSE_MEM) {
            const int e = a.n_ev + s;  // n - rank
            const double w = a.lam_zero ? (e == 0 ? 1.0 : 0.0) : exp2((double)e * a.log2lam_d);
            u = w * (kv > 0.f ? (double)kv + 1.0 : exp((double)kv));
          } else {
            u = kv;
          }
          if (dd == 0) ++cnt;
        }
      }
      sv[tt][dd] = vv;
      su[tt][dd] = u;
    }
    if (!fuse) continue;
    __syncthreads();
    if (tid < D) {
      for (int tt = 0; tt < kTok; ++tt) { v0 += su[tt][tid]; v1 += sv[tt][tid]; }
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid + i * 256, r = e / D, col = e % D;
      double s = acc[i];
      for (int tt = 0; tt < kTok; ++tt) s = fma(sv[tt][r], su[tt][col], s);
      acc[i] = s;
    }
    __syncthreads();
  }
  if (!fuse) return;
  float* pm = a.partM + (pair * a.n_chunks + c) * (size_t)(D * D);
#pragma unroll
  for (int i = 0; i < EPT; ++i) pm[tid + i * 256] = (float)acc[i];
  float* pv = a.partv + (pair * a.n_chunks + c) * (size_t)(2 * D);
  if (tid < D) { pv[tid] = (float)v0; pv[D + tid] = (float)v1; }
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  if (cnt) atomicAdd(&s_cnt, cnt);
  __syncthreads();
  if (tid == 0) a.partn[pair * a.n_chunks + c] = s_cnt;
  if (!last_block_ticket(a.counters + pair, a.n_chunks, &s_flag)) return;
  compact_finish<D>(a, pair);
}

// ------------------------------------------------------------------ side-data gather
__global__ void gather_rows_kernel(int rows, int L, int cap, int words, const uint32_t* __restrict__ src,
                                   const int32_t* __restrict__ slot_map, uint32_t* __restrict__ dst) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)rows * L * words;
  if (i >= total) return;
  const size_t rt = i / words;
  const int w = (int)(i % words);
  const int r = (int)(rt / L), t = (int)(rt % L);
  const int s = slot_map[rt];
  if (s >= 0 && s < cap) dst[((size_t)r * cap + s) * words + w] = src[i];
}

// ------------------------------------------------------------------ rank-r update
struct MemArgs {
  const void* K;
  const void* V;
  const int32_t* row_slot;
  float* M;
  float* bvec;
  int H_kv, r, cap;
  float lam;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void mem_update_kernel(MemArgs a) {
  // grid (D*D/1024, H_kv, b): each thread updates 4 consecutive elements of one row
  const int g = blockIdx.y, bb = blockIdx.z;
  const size_t pair = (size_t)bb * a.H_kv + g;
  __shared__ float sv[32][D], su[32][D];
  const int e0 = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int row = e0 / D, col = e0 % D;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float bacc = 0.f;
  for (int r0 = 0; r0 < a.r; r0 += 32) {
    const int nr = min(32, a.r - r0);
    for (int i = threadIdx.x; i < 32 * D; i += 256) {
      const int ii = i / D, dd = i % D, ri = r0 + ii;
      float k = 0.f, v = 0.f, w = 0.f;
      const int slot = a.row_slot ? a.row_slot[bb] : 0;
      if (ii < nr && slot >= 0 && slot < (a.row_slot ? a.cap : 1)) {
        const T *kp, *vp;
        if (a.row_slot) {
          const int s = slot;
          kp = reinterpret_cast<const T*>(a.K) + (pair * a.cap + s) * D;
          vp = reinterpret_cast<const T*>(a.V) + pair * a.cap * D + s;   // dim-major V cache
          k = load_scalar<T>(kp + dd);
          v = load_scalar<T>(vp + (size_t)dd * a.cap);
        } else {
          kp = reinterpret_cast<const T*>(a.K) + (((size_t)bb * a.r + ri) * a.H_kv + g) * D;
          vp = reinterpret_cast<const T*>(a.V) + (((size_t)bb * a.r + ri) * a.H_kv + g) * D;
          k = load_scalar<T>(kp + dd);
          v = load_scalar<T>(vp + dd);
        }
        const int e = a.r - 1 - ri;  // lam^(r-i) with i = ri + 1
        w = a.lam == 0.f ? (e == 0 ? 1.f : 0.f) : __powf(a.lam, (float)e);
      }
      sv[ii][dd] = v;
      su[ii][dd] = w * phi_f(k);
    }
    __syncthreads();
    for (int ii = 0; ii < nr; ++ii) {
      const float v = sv[ii][row];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(v, su[ii][col + j], acc[j]);
    }
    if (blockIdx.x == 0 && threadIdx.x < D)
      for (int ii = 0; ii < nr; ++ii) bacc += su[ii][threadIdx.x];
    __syncthreads();
  }
  const float dec = a.lam == 0.f ? (a.r == 0 ? 1.f : 0.f) : __powf(a.lam, (float)a.r);
  float* Mp = a.M + pair * D * D + (size_t)row * D + col;
  float4 m = *reinterpret_cast<float4*>(Mp);
  m.x = fmaf(dec, m.x, acc[0]); m.y = fmaf(dec, m.y, acc[1]);
  m.z = fmaf(dec, m.z, acc[2]); m.w = fmaf(dec, m.w, acc[3]);
  *reinterpret_cast<float4*>(Mp) = m;
  if (blockIdx.x == 0 && threadIdx.x < D) {
    float* bp = a.bvec + pair * D + threadIdx.x;
    *bp = fmaf(dec, *bp, bacc);
  }
}

struct CompactWs { size_t cnt, M, v, n, total; };
static int compact_chunk(const kvm_compact_desc* d) {
  // ~4 chunks per (sequence, KV head) for long rows, whole row for short ones
  int ch = (d->L + 3) / 4;
  ch = std::max(ch, 1024);
  ch = (ch + kTok - 1) / kTok * kTok;
  return ch;
}
static CompactWs compact_ws(const kvm_compact_desc* d) {
  const size_t pairs = (size_t)d->b * d->H_kv;
  const int ch = compact_chunk(d);
  const size_t nc = (d->L + ch - 1) / ch;
  CompactWs w;
  w.cnt = 0;
  w.M = kCounterBytes;
  w.v = align_up(w.M + pairs * nc * d->d * d->d * sizeof(float), 256);
  w.n = align_up(w.v + pairs * nc * 2 * d->d * sizeof(float), 256);
  w.total = align_up(w.n + pairs * nc * sizeof(int), 256);
  return w;
}

}  // namespace kvm

using namespace kvm;

extern "C" size_t kvm_compact_workspace_size(const kvm_compact_desc* d) {
  if (!d || d->b <= 0 || d->L <= 0 || d->H_kv <= 0 || d->d <= 0) return 0;
  return compact_ws(d).total;
}

extern "C" kvm_status kvm_compact_kv(const kvm_compact_desc* d, const void* K, const void* V,
                                     const int32_t* slot_map, void* Kc, void* Vc, float* M, float* bvec,
                                     int32_t* n_e, float* s_k, float* s_v, float* S, void* ws,
                                     size_t ws_bytes, void* stream) {
  KVM_PTR(d);
  KVM_REQUIRE(d->b > 0 && d->L > 0 && d->H_kv > 0, KVM_ERR_SHAPE, "b, L, H_kv must be positive");
  KVM_REQUIRE(d->d == 64 || d->d == 128, KVM_ERR_SHAPE, "head dim %d not in {64, 128}", d->d);
  KVM_REQUIRE(d->dtype == KVM_F32 || d->dtype == KVM_BF16, KVM_ERR_DTYPE, "dtype %d", d->dtype);
  KVM_REQUIRE(d->flags == 0 || d->flags == KVM_FUSE_MEM || d->flags == KVM_FUSE_MOMENTS, KVM_ERR_RANGE,
              "flags %d", d->flags);
  KVM_REQUIRE(d->keep >= 0 && d->keep <= d->L, KVM_ERR_RANGE, "keep %d outside [0, L]", d->keep);
  KVM_REQUIRE(d->lam >= 0.f && d->lam <= 1.f, KVM_ERR_RANGE, "lam %g outside [0, 1]", d->lam);
  KVM_REQUIRE((Kc == nullptr) == (Vc == nullptr), KVM_ERR_NULL, "Kc and Vc must both be given or both NULL");
  KVM_REQUIRE(Kc == nullptr || d->cap >= d->keep, KVM_ERR_RANGE, "cap %d below keep %d", d->cap, d->keep);
  KVM_PTR_ALIGNED(K); KVM_PTR_ALIGNED(V); KVM_PTR_ALIGNED(slot_map);
  KVM_OPT_ALIGNED(Kc); KVM_OPT_ALIGNED(Vc);
  if (d->flags == KVM_FUSE_MEM) { KVM_PTR_ALIGNED(M); KVM_PTR_ALIGNED(bvec); }
  if (d->flags == KVM_FUSE_MOMENTS) {
    KVM_PTR_ALIGNED(n_e); KVM_PTR_ALIGNED(s_k); KVM_PTR_ALIGNED(s_v); KVM_PTR_ALIGNED(S);
  }
  KVM_REQUIRE((size_t)d->b * d->H_kv <= (size_t)kMaxCounters, KVM_ERR_SHAPE, "b * H_kv exceeds %d", kMaxCounters);
  const CompactWs w = compact_ws(d);
  if (d->flags) {
    KVM_REQUIRE(ws != nullptr && ws_bytes >= w.total, KVM_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
    KVM_ALIGNED(ws);
  }
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;

  CompactArgs a{};
  a.K = K; a.V = V; a.slot_map = slot_map; a.Kc = Kc; a.Vc = Vc;
  if (d->flags == KVM_FUSE_MEM) { a.M = M; a.vec0 = bvec; }
  if (d->flags == KVM_FUSE_MOMENTS) { a.M = S; a.vec0 = s_k; a.vec1 = s_v; a.n_e = n_e; }
  char* base = static_cast<char*>(ws);
  if (d->flags) {
    a.counters = reinterpret_cast<int*>(base + w.cnt);
    a.partM = reinterpret_cast<float*>(base + w.M);
    a.partv = reinterpret_cast<float*>(base + w.v);
    a.partn = reinterpret_cast<int*>(base + w.n);
  }
  a.L = d->L; a.H_kv = d->H_kv; a.cap = d->cap; a.per_head = d->per_head;
  a.n_ev = d->L - d->keep;
  a.chunk = compact_chunk(d);
  a.n_chunks = (d->L + a.chunk - 1) / a.chunk;
  if (d->kv_head_major) {
    a.tok_stride = d->d; a.head_stride = (long long)d->L * d->d; a.batch_stride = (long long)d->H_kv * d->L * d->d;
  } else {
    a.tok_stride = (long long)d->H_kv * d->d; a.head_stride = d->d; a.batch_stride = (long long)d->L * d->H_kv * d->d;
  }
  a.mode = d->flags;
  a.lam_zero = d->lam == 0.f;
  a.log2lam = d->lam > 0.f ? (float)log2((double)d->lam) : 0.f;
  a.log2lam_d = d->lam > 0.f ? log2((double)d->lam) : 0.0;
  a.lam_n = (float)pow((double)d->lam, (double)a.n_ev);
  dim3 grid(a.n_chunks, d->H_kv, d->b);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->dtype == KVM_BF16) {
    if (d->d == 128) hipLaunchKernelGGL(compact_mfma_kernel<128>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(compact_mfma_kernel<64>, grid, dim3(256), 0, s, a);
  } else {
    if (d->d == 128) hipLaunchKernelGGL(compact_f32_kernel<128>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(compact_f32_kernel<64>, grid, dim3(256), 0, s, a);
  }
  return check_hip(hipGetLastError(), "compact kernel launch");
}

extern "C" kvm_status kvm_gather_rows(int32_t rows, int32_t L, int32_t cap, int32_t elem_bytes, const void* src,
                                      const int32_t* slot_map, void* dst, void* stream) {
  KVM_REQUIRE(rows > 0 && L > 0 && cap > 0, KVM_ERR_SHAPE, "rows, L, cap must be positive");
  KVM_REQUIRE(elem_bytes > 0 && elem_bytes % 4 == 0, KVM_ERR_SHAPE, "elem_bytes %d not a positive multiple of 4", elem_bytes);
  KVM_PTR_ALIGNED(src); KVM_PTR_ALIGNED(slot_map); KVM_PTR_ALIGNED(dst);
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;
  const int words = elem_bytes / 4;
  const size_t total = (size_t)rows * L * words;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), rows, L, cap, words, static_cast<const uint32_t*>(src),
                     slot_map, static_cast<uint32_t*>(dst));
  return check_hip(hipGetLastError(), "gather_rows launch");
}

extern "C" kvm_status kvm_mem_update(const kvm_mem_desc* d, const void* K_rows, const void* V_rows,
                                     const int32_t* row_slot, float* M, float* bvec, void* stream) {
  KVM_PTR(d);
  KVM_REQUIRE(d->b > 0 && d->H_kv > 0 && d->r >= 0, KVM_ERR_SHAPE, "b, H_kv positive and r >= 0 required");
  KVM_REQUIRE(d->d == 64 || d->d == 128, KVM_ERR_SHAPE, "head dim %d not in {64, 128}", d->d);
  KVM_REQUIRE(d->dtype == KVM_F32 || d->dtype == KVM_BF16, KVM_ERR_DTYPE, "dtype %d", d->dtype);
  KVM_REQUIRE(d->lam >= 0.f && d->lam <= 1.f, KVM_ERR_RANGE, "lam %g outside [0, 1]", d->lam);
  KVM_REQUIRE(row_slot == nullptr || (d->r == 1 && d->cap > 0), KVM_ERR_RANGE, "row_slot needs r == 1 and cap > 0");
  KVM_PTR_ALIGNED(K_rows); KVM_PTR_ALIGNED(V_rows); KVM_PTR_ALIGNED(M); KVM_PTR_ALIGNED(bvec);
  KVM_OPT_ALIGNED(row_slot);
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;
  if (d->r == 0) return KVM_OK;
  MemArgs a{K_rows, V_rows, row_slot, M, bvec, d->H_kv, d->r, d->cap, d->lam};
  dim3 grid(d->d * d->d / 1024, d->H_kv, d->b);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->dtype == KVM_BF16) {
    if (d->d == 128) hipLaunchKernelGGL((mem_update_kernel<uint16_t, 128>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((mem_update_kernel<uint16_t, 64>), grid, dim3(256), 0, s, a);
  } else {
    if (d->d == 128) hipLaunchKernelGGL((mem_update_kernel<float, 128>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((mem_update_kernel<float, 64>), grid, dim3(256), 0, s, a);
  }
  return check_hip(hipGetLastError(), "mem_update launch");
}
