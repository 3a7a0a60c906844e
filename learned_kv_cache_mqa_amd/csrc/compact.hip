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
// fp32 inputs use fp32 FMA.  Partial states per chunk go to the workspace; a second kernel
// sums them in chunk order (deterministic, no float atomics) and applies the decay of the
// previous state: M <- lam^n M + sum_c M_c.
#include "common.hpp"

namespace kvm {

struct CompactArgs {
  const void* K;
  const void* V;
  const int32_t* slot_map;
  float* M;     // memory: M; moments: S
  float* vec0;  // memory: bvec; moments: s_k
  float* vec1;  // moments: s_v
  int32_t* n_e;
  float* partM;    // [pairs, chunks, D, D]
  float* partv;    // [pairs, chunks, 2, D]
  int* partn;      // [pairs, chunks]
  int L, H_kv, n_ev, chunk, n_chunks, per_head;
  long long tok_stride, head_stride, batch_stride;  // elements
  int mode;        // 0 copy, KVM_FUSE_MEM, KVM_FUSE_MOMENTS
  float log2lam;   // log2(lam) (lam > 0)
  double log2lam_d;
  int lam_zero;    // lam == 0
  float lam_n;     // lam^n_ev
};

// ------------------------------------------------------------------ fixed-order reduce
// grid (ceil(E / 1024), pairs) with E = D*D + 2*D + 1 elements per (sequence, KV head):
// sums the chunk partials in chunk order (deterministic) and applies the decay of the
// previous state: state <- lam^n state + sum_c part_c (lam^n = 1 for the moment sums).
template <int D>
__global__ __launch_bounds__(256) void compact_reduce_kernel(CompactArgs a) {
  const size_t pair = blockIdx.y;
  const int e0 = (blockIdx.x * 256 + threadIdx.x) * 4;
  const bool mem = a.mode == KVM_FUSE_MEM;
  const float dec = mem ? a.lam_n : 1.f;
  if (e0 < D * D) {
    const float* pm = a.partM + pair * a.n_chunks * (size_t)(D * D) + e0;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < a.n_chunks; ++c) {
      const float4 v = *reinterpret_cast<const float4*>(pm + (size_t)c * D * D);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    float4* mo = reinterpret_cast<float4*>(a.M + pair * (size_t)(D * D) + e0);
    float4 o = *mo;
    o.x = fmaf(dec, o.x, acc.x); o.y = fmaf(dec, o.y, acc.y);
    o.z = fmaf(dec, o.z, acc.z); o.w = fmaf(dec, o.w, acc.w);
    *mo = o;
  } else if (e0 < D * D + 2 * D) {
    const int i = e0 - D * D;
    if (mem && i >= D) return;
    const float* pv = a.partv + pair * a.n_chunks * (size_t)(2 * D) + i;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < a.n_chunks; ++c) {
      const float4 v = *reinterpret_cast<const float4*>(pv + (size_t)c * 2 * D);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    float4* vo = reinterpret_cast<float4*>((i < D ? a.vec0 : a.vec1) + pair * D + (i % D));
    float4 o = *vo;
    o.x = fmaf(dec, o.x, acc.x); o.y = fmaf(dec, o.y, acc.y);
    o.z = fmaf(dec, o.z, acc.z); o.w = fmaf(dec, o.w, acc.w);
    *vo = o;
  } else if (e0 == D * D + 2 * D && !mem) {
    int n = 0;
    for (int c = 0; c < a.n_chunks; ++c) n += a.partn[pair * a.n_chunks + c];
    a.n_e[pair] += n;
  }
}

// ------------------------------------------------------------------ bf16: matrix cores
// LDS tile: per dim row, 16 token pairs (32 tokens, bf16x2 per word) + 2 pad words.  The
// pair words of a row sit in four groups of four (the 8 tokens an MFMA lane reads); the groups
// are XOR-swizzled by the row's 32-dim tile index.  With the pitch of 18 words this keeps
// both the transposed stores (a wave's 64 lanes: 16 dim blocks x 4 token pairs of one group)
// and the 8-byte fragment loads (32 consecutive rows) free of bank conflicts.
constexpr int kTok = 32;
constexpr int kPitch = 18;
__device__ __forceinline__ int pair_word(int row, int pr) { return row * kPitch + (pr ^ (((row >> 5) & 3) << 2)); }

// Stages one tile of 32 tokens for the contraction: this thread holds tokens (2 pr, 2 pr + 1)
// x dims db*8 .. db*8+8 of K and V.  Writes V^T (exact bf16) to sV and u = w phi(k) (memory)
// or k (moments) to sH (+ the bf16 remainder of u to sL in memory mode), one word per token
// pair per dim row; rows of kept tokens and positions past the chunk are staged as zeros.
//   memory: w = lam^(n - rank) = 2^lw,  w phi(x) = w (x + 1) for x > 0, 2^(x log2 e + lw) else.
template <int D, bool MEM>
__device__ __forceinline__ void stage_tile(const CompactArgs& a, int pr, int db, bool loader,
                                           int t0, int p1, uint4 k0v, uint4 k1v, uint4 v0v, uint4 v1v,
                                           int s0, int s1, uint32_t* sV, uint32_t* sH, uint32_t* sL,
                                           float (&vacc0)[8], float (&vacc1)[8], int& nloc) {
  const bool ev0 = loader && t0 < p1 && s0 < 0;
  const bool ev1 = loader && t0 + 1 < p1 && s1 < 0;
  if (db == 0) nloc += (int)ev0 + (int)ev1;
  if (!loader) return;   // D = 64: the spare threads alias a loader's LDS words
  float w0 = 0.f, w1 = 0.f, lw0 = -INFINITY, lw1 = -INFINITY;
  if (MEM) {
    const int e0 = a.n_ev + s0, e1 = a.n_ev + s1;
    if (ev0) lw0 = a.lam_zero ? (e0 == 0 ? 0.f : -INFINITY) : (float)e0 * a.log2lam;
    if (ev1) lw1 = a.lam_zero ? (e1 == 0 ? 0.f : -INFINITY) : (float)e1 * a.log2lam;
    w0 = __builtin_amdgcn_exp2f(lw0);
    w1 = __builtin_amdgcn_exp2f(lw1);
  }
  // byte selectors: a token's bf16 half of a K word moved to the top half (or zero when the
  // token is not evicted), and the two tokens' halves of a V word packed into one word
  const uint32_t se0 = ev0 ? 0x01000c0cu : 0x0c0c0c0cu, so0 = ev0 ? 0x03020c0cu : 0x0c0c0c0cu;
  const uint32_t se1 = ev1 ? 0x01000c0cu : 0x0c0c0c0cu, so1 = ev1 ? 0x03020c0cu : 0x0c0c0c0cu;
  const uint32_t vmask = (ev0 ? 0x0000ffffu : 0u) | (ev1 ? 0xffff0000u : 0u);
  const uint32_t k0[4] = {k0v.x, k0v.y, k0v.z, k0v.w}, k1[4] = {k1v.x, k1v.y, k1v.z, k1v.w};
  const uint32_t v0[4] = {v0v.x, v0v.y, v0v.z, v0v.w}, v1[4] = {v1v.x, v1v.y, v1v.z, v1v.w};
  constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int at = pair_word(db * 8 + e, pr);
    const bool odd = e & 1;
    const uint32_t vw = __builtin_amdgcn_perm(v1[e >> 1], v0[e >> 1], odd ? 0x07060302u : 0x05040100u) & vmask;
    sV[at] = vw;
    const float x0 = __uint_as_float(__builtin_amdgcn_perm(0u, k0[e >> 1], odd ? so0 : se0));
    const float x1 = __uint_as_float(__builtin_amdgcn_perm(0u, k1[e >> 1], odd ? so1 : se1));
    f32x2_t u;
    if (MEM) {
      const float n0 = __builtin_amdgcn_exp2f(fmaf(x0, kLog2e, lw0));
      const float n1 = __builtin_amdgcn_exp2f(fmaf(x1, kLog2e, lw1));
      u.x = x0 > 0.f ? fmaf(w0, x0, w0) : n0;
      u.y = x1 > 0.f ? fmaf(w1, x1, w1) : n1;
    } else {
      u.x = x0;
      u.y = x1;
      vacc1[e] += __uint_as_float(vw << 16) + __uint_as_float(vw & 0xffff0000u);
    }
    vacc0[e] += u.x + u.y;
    const bf16x2_t hi = __builtin_convertvector(u, bf16x2_t);   // round to nearest even
    uint32_t hw;
    __builtin_memcpy(&hw, &hi, 4);
    sH[at] = hw;
    if (MEM) {
      f32x2_t r;
      r.x = u.x - __uint_as_float(hw << 16);
      r.y = u.y - __uint_as_float(hw & 0xffff0000u);
      const bf16x2_t lo = __builtin_convertvector(r, bf16x2_t);
      uint32_t lw;
      __builtin_memcpy(&lw, &lo, 4);
      sL[at] = lw;
    }
  }
}

constexpr int kCompactNB = 2;    // K/V tiles in flight per wave (register ring depth)
constexpr int kCompactWPE = 2;   // waves per SIMD the kernel is compiled for
// Contraction of the evicted rows of one chunk of positions of one (sequence, KV head):
// grid (chunks, H_kv, b), 256 threads.  Raw K/V rows stream through a register ring NB tiles
// deep; staged tiles alternate between two LDS buffers so that the staging of tile t + 1 (VALU)
// overlaps the matrix-core work on tile t, with one barrier per tile.  Each wave owns a
// 2 x 2 block of 32 x 32 output tiles (D = 128) or one tile (D = 64).
template <int D, bool MEM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kCompactWPE, kCompactWPE)))
void compact_mfma_kernel(CompactArgs a) {
  static_assert(D == 64 || D == 128, "D");
  constexpr int NT = D / 32;               // 32x32 tiles per side
  constexpr int NTI = NT / 2, NTJ = NT / 2; // tiles per wave along v rows / u columns
  constexpr int DB = D / 8;                // 8-dim blocks per row
  constexpr int PAIRS = (256 / DB) < (kTok / 2) ? (256 / DB) : (kTok / 2);
  static_assert(PAIRS == kTok / 2, "one pass of token pairs per tile");
  constexpr int NB = kCompactNB;       // raw tiles in flight per thread
  const int c = blockIdx.x, g = blockIdx.y, bb = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t pair = (size_t)bb * a.H_kv + g;

  __shared__ uint32_t sV[2][D * kPitch];
  __shared__ uint32_t sH[2][D * kPitch];
  __shared__ uint32_t sL[2][MEM ? D * kPitch : 1];
  __shared__ int s_n;

  const int p0 = c * a.chunk, p1 = min(a.L, p0 + a.chunk);
  const int ntiles = (p1 - p0 + kTok - 1) / kTok;
  // this chunk's rows through buffer resources: positions past p1 read as zeros (slot 0,
  // i.e. kept, so they stage nothing)
  const long long cbase = bb * a.batch_stride + g * a.head_stride + (long long)p0 * a.tok_stride;
  const int rowb = (int)(a.tok_stride * 2);
  const int nbytes = (p1 - p0 - 1) * rowb + D * 2;
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(reinterpret_cast<const uint16_t*>(a.K) + cbase, nbytes);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(reinterpret_cast<const uint16_t*>(a.V) + cbase, nbytes);
  const __amdgpu_buffer_rsrc_t rS =
      make_rsrc(a.slot_map + (a.per_head ? pair : (size_t)bb) * a.L + p0, (p1 - p0) * 4);

  // thread -> (token pair, 8-dim block), dim blocks fastest: 16 lanes read one token's whole
  // 256-byte row.  D = 64 leaves half the threads without a slot of their own (they load a
  // duplicate and stage nothing)
  const int db = tid % DB;
  const int pr = (tid / DB) % PAIRS;
  const bool loader = DB * PAIRS >= 256 || tid / PAIRS < DB;
  float vacc0[8], vacc1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { vacc0[e] = 0.f; vacc1[e] = 0.f; }
  int nloc = 0;

  const int wi = wave / 2, wj = wave % 2;
  f32x16_t acc[NTI * NTJ];
#pragma unroll
  for (int t = 0; t < NTI * NTJ; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[t][j] = 0.f;

  uint4 rk[NB][2] = {}, rv[NB][2] = {};
  int rs[NB][2] = {};
  // Loads are unconditional and the tile loop runs a multiple of NB tiles without an early
  // exit, so the number of loads in flight is static and the waits cover only the oldest tile.
  const int voff0 = 2 * pr * rowb + db * 16;
  auto fetch = [&](int st, int tile) {
    const int tb = tile * kTok * rowb;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int off = voff0 + h * rowb + tb;
      rs[st][h] = __builtin_amdgcn_raw_buffer_load_b32(rS, (tile * kTok + 2 * pr + h) * 4, 0, 0);
      const auto kv = __builtin_amdgcn_raw_buffer_load_b128(rK, off, 0, 0);
      const auto vv = __builtin_amdgcn_raw_buffer_load_b128(rV, off, 0, 0);
      rk[st][h] = make_uint4(kv[0], kv[1], kv[2], kv[3]);
      rv[st][h] = make_uint4(vv[0], vv[1], vv[2], vv[3]);
    }
  };
#pragma unroll
  for (int st = 0; st < NB; ++st) fetch(st, st);
  stage_tile<D, MEM>(a, pr, db, loader, p0 + 2 * pr, p1, rk[0][0], rk[0][1], rv[0][0], rv[0][1], rs[0][0], rs[0][1],
                     sV[0], sH[0], sL[0], vacc0, vacc1, nloc);
  fetch(0, NB);
  __syncthreads();

  static_assert(NB % 2 == 0, "LDS buffer parity follows the ring slot");
  for (int t0 = 0; t0 < ntiles; t0 += NB) {
#pragma unroll
    for (int st = 0; st < NB; ++st) {
      const int t = t0 + st;   // tiles past the chunk stage zeros and add nothing
      const int cur = st & 1, nxt = cur ^ 1;
      // matrix cores on tile t: 2 k-steps of 16 tokens; lane (m, kg) reads 8 tokens = 4 words.
      // All hi products are issued before the lo ones so that no MFMA waits on the previous.
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int grp = ks * 2 + (lane >> 5);   // this lane's group of 4 pair words
        const int m = lane & 31;
        bf16x8_t A[NTI], Bh[NTJ], Bl[NTJ];
#pragma unroll
        for (int x = 0; x < NTI; ++x) {
          const int ti = wi * NTI + x;
          const uint32_t* pa = sV[cur] + (ti * 32 + m) * kPitch + ((grp ^ (ti & 3)) << 2);
          const uint2 a0 = *reinterpret_cast<const uint2*>(pa), a1 = *reinterpret_cast<const uint2*>(pa + 2);
          const uint4 av = {a0.x, a0.y, a1.x, a1.y};
          __builtin_memcpy(&A[x], &av, 16);
        }
#pragma unroll
        for (int y = 0; y < NTJ; ++y) {
          const int tj = wj * NTJ + y;
          const int r = (tj * 32 + m) * kPitch + ((grp ^ (tj & 3)) << 2);
          const uint2 h0 = *reinterpret_cast<const uint2*>(sH[cur] + r), h1 = *reinterpret_cast<const uint2*>(sH[cur] + r + 2);
          const uint4 hv = {h0.x, h0.y, h1.x, h1.y};
          __builtin_memcpy(&Bh[y], &hv, 16);
          if (MEM) {
            const uint2 l0 = *reinterpret_cast<const uint2*>(sL[cur] + r), l1 = *reinterpret_cast<const uint2*>(sL[cur] + r + 2);
            const uint4 lv = {l0.x, l0.y, l1.x, l1.y};
            __builtin_memcpy(&Bl[y], &lv, 16);
          }
        }
#pragma unroll
        for (int x = 0; x < NTI; ++x)
#pragma unroll
          for (int y = 0; y < NTJ; ++y)
            acc[x * NTJ + y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[x], Bh[y], acc[x * NTJ + y], 0, 0, 0);
        if (MEM)
#pragma unroll
          for (int x = 0; x < NTI; ++x)
#pragma unroll
            for (int y = 0; y < NTJ; ++y)
              acc[x * NTJ + y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[x], Bl[y], acc[x * NTJ + y], 0, 0, 0);
      }
      // stage tile t + 1 (ring slot (st + 1) % NB) into the other buffer, refill its slot
      const int sn = (st + 1) % NB;
      stage_tile<D, MEM>(a, pr, db, loader, p0 + (t + 1) * kTok + 2 * pr, p1, rk[sn][0], rk[sn][1], rv[sn][0],
                         rv[sn][1], rs[sn][0], rs[sn][1], sV[nxt], sH[nxt], sL[nxt], vacc0, vacc1, nloc);
      fetch(sn, t + 1 + NB);
      __syncthreads();
    }
  }

  // partial state of this chunk -> workspace
  float* pm = a.partM + (pair * a.n_chunks + c) * (size_t)(D * D);
#pragma unroll
  for (int x = 0; x < NTI; ++x)
#pragma unroll
    for (int y = 0; y < NTJ; ++y) {
      const int ti = wi * NTI + x, tj = wj * NTJ + y;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = ti * 32 + 8 * (j / 4) + 4 * (lane / 32) + (j % 4);
        const int col = tj * 32 + (lane & 31);
        pm[r * D + col] = acc[x * NTJ + y][j];
      }
    }
  // vector sums over the token pairs: in LDS (the tiles are free now), then thread i < 2D sums
  // entry i over the pairs in order
  __syncthreads();
  float* sv = reinterpret_cast<float*>(sV[0]);   // [PAIRS][2D] floats
  static_assert(PAIRS * 2 * D <= 2 * D * kPitch, "vector sums fit in one staged tile");
  if (loader) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[pr * 2 * D + db * 8 + e] = vacc0[e];
      sv[pr * 2 * D + D + db * 8 + e] = vacc1[e];
    }
  }
  if (tid == 0) s_n = 0;
  __syncthreads();
  float* pv = a.partv + (pair * a.n_chunks + c) * (size_t)(2 * D);
  for (int i = tid; i < 2 * D; i += 256) {
    float x = 0.f;
    for (int q = 0; q < PAIRS; ++q) x += sv[q * 2 * D + i];
    pv[i] = x;
  }
  if (db == 0 && nloc) atomicAdd(&s_n, nloc);
  __syncthreads();
  if (tid == 0) a.partn[pair * a.n_chunks + c] = s_n;
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
  __shared__ int s_cnt;
  const float* Kb = reinterpret_cast<const float*>(a.K) + bb * a.batch_stride + g * a.head_stride;
  const float* Vb = reinterpret_cast<const float*>(a.V) + bb * a.batch_stride + g * a.head_stride;
  const int32_t* smr = a.slot_map + (a.per_head ? pair : (size_t)bb) * a.L;
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
        if (s < 0) {
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
}

// ------------------------------------------------------------------ kept-row gather (A5)
// Kept rows into the caches: slot s of row r holds position idx[r, s].  grid
// (ceil(keep / 64), H_kv, b), 256 threads; a block moves 64 slots.  K rows are copied in
// 16-byte pieces; V rows are transposed through LDS so that each dim row of the dim-major
// V cache is written as one contiguous run of 64 slots.
struct GatherArgs {
  const void* K;
  const void* V;
  const int32_t* idx;
  void* Kc;
  void* Vc;
  int L, H_kv, cap, keep, per_head, v_row_major;
  long long tok_stride, head_stride, batch_stride;  // elements
};

template <typename T, int D>
__global__ __launch_bounds__(256) void gather_kv_kernel(GatherArgs a) {
  constexpr int E16 = 16 / (int)sizeof(T);   // elements per 16-byte piece
  constexpr int C16 = D / E16;               // pieces per row
  constexpr int SP = 64 + 4 / (int)sizeof(T); // LDS pitch (elements): odd word stride
  const int g = blockIdx.y, bb = blockIdx.z, tid = threadIdx.x;
  const size_t pair = (size_t)bb * a.H_kv + g;
  const int s0 = blockIdx.x * 64;
  const int ns = min(64, a.keep - s0);
  __shared__ T sVt[D * SP];
  __shared__ int sPos[64];
  const int32_t* ix = a.idx + (a.per_head ? pair : (size_t)bb) * a.keep + s0;
  if (tid < ns) {
    const int t = ix[tid];
    sPos[tid] = (t >= 0 && t < a.L) ? t : -1;   // an out-of-range index copies nothing
  }
  __syncthreads();
  const T* Kb = reinterpret_cast<const T*>(a.K) + bb * a.batch_stride + g * a.head_stride;
  const T* Vb = reinterpret_cast<const T*>(a.V) + bb * a.batch_stride + g * a.head_stride;
  T* Kcb = reinterpret_cast<T*>(a.Kc) + (pair * a.cap + s0) * D;
  T* Vcb = reinterpret_cast<T*>(a.Vc) + pair * a.cap * D + s0;
  // every load of the thread first, then the stores: in one loop each iteration's loads
  // would wait for the previous iteration's stores (the compiler cannot rule out aliasing)
  constexpr int IT = (64 * C16 + 255) / 256;   // 16-byte pieces per thread
  uint4 kv[IT], vv[IT];
#pragma unroll
  for (int r = 0; r < IT; ++r) {
    const int i = tid + r * 256;
    kv[r] = vv[r] = make_uint4(0, 0, 0, 0);
    const int t = i < ns * C16 ? sPos[i / C16] : -1;
    if (t >= 0) {
      kv[r] = *reinterpret_cast<const uint4*>(Kb + t * a.tok_stride + (i % C16) * E16);
      vv[r] = *reinterpret_cast<const uint4*>(Vb + t * a.tok_stride + (i % C16) * E16);
    }
  }
#pragma unroll
  for (int r = 0; r < IT; ++r) {
    const int i = tid + r * 256;
    if (i >= ns * C16) continue;
    const int sl = i / C16, cc = i % C16;
    *reinterpret_cast<uint4*>(Kcb + (size_t)sl * D + cc * E16) = kv[r];
    if (a.v_row_major) {   // Vc [b, H_kv, cap, d]
      *reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.Vc) + (pair * a.cap + s0 + sl) * D + cc * E16) = vv[r];
      continue;
    }
    T ve[E16];
    __builtin_memcpy(ve, &vv[r], 16);
#pragma unroll
    for (int e = 0; e < E16; ++e) sVt[(cc * E16 + e) * SP + sl] = ve[e];
  }
  if (a.v_row_major) return;   // block-uniform
  __syncthreads();
  // dim-major rows out in 16-byte pieces of E16 consecutive slots, aligned when cap is a
  // multiple of E16 (s0 is a multiple of 64); otherwise, and for a piece past the block's last
  // slot, element by element
  constexpr int PPR = 64 / E16;   // pieces per dim row
  const bool vec = a.cap % E16 == 0;
  for (int i = tid; i < D * PPR; i += 256) {
    const int dim = i / PPR, sl = (i % PPR) * E16;
    if (sl >= ns) continue;
    T ve[E16];
#pragma unroll
    for (int e = 0; e < E16; ++e) ve[e] = sVt[dim * SP + sl + e];
    if (vec && sl + E16 <= ns) {
      uint4 w;
      __builtin_memcpy(&w, ve, 16);
      *reinterpret_cast<uint4*>(Vcb + (size_t)dim * a.cap + sl) = w;
    } else {
#pragma unroll
      for (int e = 0; e < E16; ++e)
        if (sl + e < ns) Vcb[(size_t)dim * a.cap + sl + e] = ve[e];
    }
  }
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
// Latent memory (MOM = false): M <- lam^r M + sum_i lam^(r-i) v_i phi(k_i)^T, bvec likewise.
// Moments (MOM = true): S += sum_i v_i k_i^T, s_k (in bvec) += sum k, s_v += sum v,
// n_e += r.  Rows are summed in order i = 1 .. r (deterministic).
struct MemArgs {
  const void* K;
  const void* V;
  const int32_t* row_slot;
  float* M;      // M, or S
  float* bvec;   // bvec, or s_k
  int H_kv, r, cap;
  float lam;
  float* s_v;    // moments only
  int32_t* n_e;  // moments only
};

template <typename T, int D, bool MOM>
__global__ __launch_bounds__(256) void mem_update_kernel(MemArgs a) {
  // grid (D*D/1024, H_kv, b): each thread updates 4 consecutive elements of one row
  const int g = blockIdx.y, bb = blockIdx.z;
  const size_t pair = (size_t)bb * a.H_kv + g;
  if (a.row_slot && (a.row_slot[bb] < 0 || a.row_slot[bb] >= a.cap)) return;   // nothing evicted
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
        w = MOM ? 1.f : a.lam == 0.f ? (e == 0 ? 1.f : 0.f) : __powf(a.lam, (float)e);
      }
      sv[ii][dd] = v;
      su[ii][dd] = MOM ? w * k : w * phi_f(k);
    }
    __syncthreads();
    for (int ii = 0; ii < nr; ++ii) {
      const float v = sv[ii][row];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(v, su[ii][col + j], acc[j]);
    }
    if (blockIdx.x == 0 && threadIdx.x < D)
      for (int ii = 0; ii < nr; ++ii) bacc += su[ii][threadIdx.x];
    if (MOM && blockIdx.x == 0 && threadIdx.x >= D && threadIdx.x < 2 * D)
      for (int ii = 0; ii < nr; ++ii) bacc += sv[ii][threadIdx.x - D];
    __syncthreads();
  }
  const float dec = MOM ? 1.f : a.lam == 0.f ? (a.r == 0 ? 1.f : 0.f) : __powf(a.lam, (float)a.r);
  float* Mp = a.M + pair * D * D + (size_t)row * D + col;
  float4 m = *reinterpret_cast<float4*>(Mp);
  m.x = fmaf(dec, m.x, acc[0]); m.y = fmaf(dec, m.y, acc[1]);
  m.z = fmaf(dec, m.z, acc[2]); m.w = fmaf(dec, m.w, acc[3]);
  *reinterpret_cast<float4*>(Mp) = m;
  if (blockIdx.x == 0 && threadIdx.x < D) {
    float* bp = a.bvec + pair * D + threadIdx.x;
    *bp = fmaf(dec, *bp, bacc);
  }
  if (MOM && blockIdx.x == 0 && threadIdx.x >= D && threadIdx.x < 2 * D) a.s_v[pair * D + threadIdx.x - D] += bacc;
  if (MOM && blockIdx.x == 1 && threadIdx.x == 0) a.n_e[pair] += a.r;   // grid.x = D D / 1024 >= 4
}

struct CompactWs { size_t M, v, n, total; };
static int compact_chunk(const kvm_compact_desc* d) {
  // 2048-token chunks: enough blocks to fill the chip at 16K tokens x 64 (sequence, KV head)
  // pairs while keeping the fp32 partial states (d*d floats per chunk) near a tenth of the
  // K/V bytes read.  Shorter inputs (a chunked prefill's pool + chunk, small batches) halve
  // the chunk, down to 512 tokens, until every CU (256) has a block.
  const long long pairs = (long long)d->b * d->H_kv;
  int ch = 2048;
  while (ch > 512 && pairs * ((d->L + ch - 1) / ch) < 256) ch /= 2;
  return ch;
}
static CompactWs compact_ws(const kvm_compact_desc* d) {
  const size_t pairs = (size_t)d->b * d->H_kv;
  const int ch = compact_chunk(d);
  const size_t nc = (d->L + ch - 1) / ch;
  CompactWs w;
  w.M = 0;
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
                                     const int32_t* slot_map, const int32_t* idx, void* Kc, void* Vc,
                                     float* M, float* bvec,
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
  KVM_REQUIRE(Kc == nullptr || idx != nullptr, KVM_ERR_NULL, "idx is required to fill the caches");
  KVM_PTR_ALIGNED(K); KVM_PTR_ALIGNED(V);
  if (d->flags) KVM_PTR_ALIGNED(slot_map);
  KVM_OPT_ALIGNED(Kc); KVM_OPT_ALIGNED(Vc);
  if (Kc) KVM_PTR_ALIGNED(idx);
  if (d->flags == KVM_FUSE_MEM) { KVM_PTR_ALIGNED(M); KVM_PTR_ALIGNED(bvec); }
  if (d->flags == KVM_FUSE_MOMENTS) {
    KVM_PTR_ALIGNED(n_e); KVM_PTR_ALIGNED(s_k); KVM_PTR_ALIGNED(s_v); KVM_PTR_ALIGNED(S);
  }
  const CompactWs w = compact_ws(d);
  if (d->flags) {
    KVM_REQUIRE(ws != nullptr && ws_bytes >= w.total, KVM_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
    KVM_ALIGNED(ws);
  }
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;

  long long tok_stride, head_stride, batch_stride;
  if (d->kv_head_major) {
    tok_stride = d->d; head_stride = (long long)d->L * d->d; batch_stride = (long long)d->H_kv * d->L * d->d;
  } else {
    tok_stride = (long long)d->H_kv * d->d; head_stride = d->d; batch_stride = (long long)d->L * d->H_kv * d->d;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = d->dtype == KVM_BF16;
  if (d->flags) {
    CompactArgs a{};
    a.K = K; a.V = V; a.slot_map = slot_map;
    if (d->flags == KVM_FUSE_MEM) { a.M = M; a.vec0 = bvec; }
    if (d->flags == KVM_FUSE_MOMENTS) { a.M = S; a.vec0 = s_k; a.vec1 = s_v; a.n_e = n_e; }
    char* base = static_cast<char*>(ws);
    a.partM = reinterpret_cast<float*>(base + w.M);
    a.partv = reinterpret_cast<float*>(base + w.v);
    a.partn = reinterpret_cast<int*>(base + w.n);
    a.L = d->L; a.H_kv = d->H_kv; a.per_head = d->per_head;
    a.n_ev = d->L - d->keep;
    a.chunk = compact_chunk(d);
    a.n_chunks = (d->L + a.chunk - 1) / a.chunk;
    a.tok_stride = tok_stride; a.head_stride = head_stride; a.batch_stride = batch_stride;
    a.mode = d->flags;
    a.lam_zero = d->lam == 0.f;
    a.log2lam = d->lam > 0.f ? (float)log2((double)d->lam) : 0.f;
    a.log2lam_d = d->lam > 0.f ? log2((double)d->lam) : 0.0;
    a.lam_n = (float)pow((double)d->lam, (double)a.n_ev);
    const dim3 grid(a.n_chunks, d->H_kv, d->b);
    const bool mem = d->flags == KVM_FUSE_MEM;
    if (bf) {
      if (d->d == 128) {
        if (mem) hipLaunchKernelGGL((compact_mfma_kernel<128, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((compact_mfma_kernel<128, false>), grid, dim3(256), 0, s, a);
      } else {
        if (mem) hipLaunchKernelGGL((compact_mfma_kernel<64, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((compact_mfma_kernel<64, false>), grid, dim3(256), 0, s, a);
      }
    } else {
      if (d->d == 128) hipLaunchKernelGGL(compact_f32_kernel<128>, grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL(compact_f32_kernel<64>, grid, dim3(256), 0, s, a);
    }
    const int E = d->d * d->d + 2 * d->d + 1;
    const dim3 rgrid((E + 1023) / 1024, d->b * d->H_kv);
    if (d->d == 128) hipLaunchKernelGGL(compact_reduce_kernel<128>, rgrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(compact_reduce_kernel<64>, rgrid, dim3(256), 0, s, a);
  }
  if (Kc && d->keep > 0) {
    GatherArgs ga{K, V, idx, Kc, Vc, d->L, d->H_kv, d->cap, d->keep, d->per_head, d->v_row_major, tok_stride,
                  head_stride, batch_stride};
    const dim3 grid((d->keep + 63) / 64, d->H_kv, d->b);
    if (bf) {
      if (d->d == 128) hipLaunchKernelGGL((gather_kv_kernel<uint16_t, 128>), grid, dim3(256), 0, s, ga);
      else hipLaunchKernelGGL((gather_kv_kernel<uint16_t, 64>), grid, dim3(256), 0, s, ga);
    } else {
      if (d->d == 128) hipLaunchKernelGGL((gather_kv_kernel<float, 128>), grid, dim3(256), 0, s, ga);
      else hipLaunchKernelGGL((gather_kv_kernel<float, 64>), grid, dim3(256), 0, s, ga);
    }
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

namespace kvm {
template <bool MOM>
static kvm_status mem_update_launch(const kvm_mem_desc* d, const MemArgs& a, hipStream_t s) {
  const dim3 grid(d->d * d->d / 1024, d->H_kv, d->b);
  if (d->dtype == KVM_BF16) {
    if (d->d == 128) hipLaunchKernelGGL((mem_update_kernel<uint16_t, 128, MOM>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((mem_update_kernel<uint16_t, 64, MOM>), grid, dim3(256), 0, s, a);
  } else {
    if (d->d == 128) hipLaunchKernelGGL((mem_update_kernel<float, 128, MOM>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((mem_update_kernel<float, 64, MOM>), grid, dim3(256), 0, s, a);
  }
  return check_hip(hipGetLastError(), MOM ? "moment_update launch" : "mem_update launch");
}
}  // namespace kvm

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
  MemArgs a{K_rows, V_rows, row_slot, M, bvec, d->H_kv, d->r, d->cap, d->lam, nullptr, nullptr};
  return mem_update_launch<false>(d, a, static_cast<hipStream_t>(stream));
}

extern "C" kvm_status kvm_moment_update(const kvm_mem_desc* d, const void* K_rows, const void* V_rows,
                                        const int32_t* row_slot, int32_t* n_e, float* s_k, float* s_v, float* S,
                                        void* stream) {
  KVM_PTR(d);
  KVM_REQUIRE(d->b > 0 && d->H_kv > 0 && d->r >= 0, KVM_ERR_SHAPE, "b, H_kv positive and r >= 0 required");
  KVM_REQUIRE(d->d == 64 || d->d == 128, KVM_ERR_SHAPE, "head dim %d not in {64, 128}", d->d);
  KVM_REQUIRE(d->dtype == KVM_F32 || d->dtype == KVM_BF16, KVM_ERR_DTYPE, "dtype %d", d->dtype);
  KVM_REQUIRE(row_slot == nullptr || (d->r == 1 && d->cap > 0), KVM_ERR_RANGE, "row_slot needs r == 1 and cap > 0");
  KVM_PTR_ALIGNED(K_rows); KVM_PTR_ALIGNED(V_rows);
  KVM_PTR_ALIGNED(n_e); KVM_PTR_ALIGNED(s_k); KVM_PTR_ALIGNED(s_v); KVM_PTR_ALIGNED(S);
  KVM_OPT_ALIGNED(row_slot);
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;
  if (d->r == 0) return KVM_OK;
  MemArgs a{K_rows, V_rows, row_slot, S, s_k, d->H_kv, d->r, d->cap, 1.f, s_v, n_e};
  return mem_update_launch<true>(d, a, static_cast<hipStream_t>(stream));
}
