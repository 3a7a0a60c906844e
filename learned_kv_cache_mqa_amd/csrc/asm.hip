// Attention-state memory (ASM) [ASM Method]: a prefix is replaced by a lookup memory of
// precomputed attention states (a, Z).
//
// Offline (calibration):
//   prefix_states_kernel   (a, lse) of every calibration query over the prefix: attention
//                          on the matrix cores, 32 queries per wave against 32-key tiles
//                          staged in LDS and shared by the block's 8 waves (heads of one
//                          KV group), online softmax in the log2 domain, P as bf16 hi + lo
//   kmeans_assign_kernel   nearest centroid per query on the matrix cores:
//                          ||c||^2 - 2 x . c with the centroids as bf16 hi + mid + lo
//   kmeans_part_kernel     per chunk of queries, every centroid's sum of its members as a
//                          one-hot contraction on the matrix cores (exact products)
//   kmeans_reduce_kernel   the chunks summed in order: the means, their planes and norms
//   state_part_kernel      per chunk of queries, every cluster's running online-softmax
//                          state of its members, rows taken in index order, in LDS
//   state_reduce_kernel    the chunk states merged in order: (a, lse - log n)
// Online (decode):
//   lookup_merge_kernel    the largest cosine similarity among a head's centroids, and the
//                          retrieved state merged with the query's local attention state
#include "common.hpp"

namespace kvm {

// ------------------------------------------------------------------ prefix states
struct PrefixArgs {
  const uint16_t* Q;   // [N, H_q, D]
  const uint16_t* K;   // prefix keys: element (t, g, c) at t * ts + g * hs + c
  const uint16_t* V;
  float* a;            // [N, H_q, D]
  float* lse;          // [N, H_q]
  int N, H_q, G, L, ts, hs;
  int acc;             // merge into the states already in a, lse (a later chunk of the prefix)
  float sl2;           // logit scale * log2(e)
};

constexpr int kPT = 32;   // keys per tile

constexpr int kPW = 8;    // waves per block (items sharing the block's K/V tiles)

// grid (ceil(G * ceil(N / 32) / kPW), H_kv), 64 kPW threads.  Wave w of block x takes item
// i = kPW x + w: query tile i / G of head g G + i % G.  At the top of step t the tile t + 1
// (loaded during step t - 1) is staged into the idle LDS buffer and tile t + 2 is loaded into
// the freed registers, so a tile's load latency spans a tile of compute.  S^T = K Q^T puts keys on the rows of
// the 32 x 32 accumulator, so each lane holds 16 keys of one query column: the row max and
// sum need one exchange between the half-waves, and the lane's probabilities are already
// the A operand of P V (with V's keys gathered in the same order from a dim-major tile).
template <int D>
__global__ __launch_bounds__(64 * kPW) void prefix_states_kernel(PrefixArgs a) {
  constexpr int KS = D / 16, NT = D / 32, NTH = 64 * kPW;
  constexpr int KP = D + 8;                  // sK row pitch (bf16)
  constexpr int VP = kPT + 8;                // sV row pitch (bf16)
  constexpr int CH = kPT * D / 8;            // 16-byte chunks per tile
  constexpr int CPT = (CH + NTH - 1) / NTH;  // chunks per thread
  __shared__ __align__(16) uint16_t sK[2][kPT * KP];
  __shared__ __align__(16) uint16_t sV[2][D * VP];
  __shared__ float sRow[kPW][kPT];
  __shared__ float sLse[kPW][kPT];

  // the wave index through readfirstlane keeps the head and the query buffer resource scalar
  const int g = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int nqt = (a.N + 31) / 32;
  const int item = blockIdx.x * kPW + wave;
  const bool active = item < a.G * nqt;
  const int h = __builtin_amdgcn_readfirstlane(g * a.G + (active ? item % a.G : 0));
  const int q0 = __builtin_amdgcn_readfirstlane((active ? item / a.G : 0) * 32);

  // B operand: lane (query q0 + col) holds dims ks * 16 + half * 8 .. + 8 (zeros past N)
  bf16x8_t qb[KS];
  {
    const auto rq = make_rsrc(a.Q + (size_t)h * D, ((a.N - 1) * a.H_q * D + D) * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = load16(rq, ((q0 + col) * a.H_q * D + ks * 16 + half * 8) * 2);
      __builtin_memcpy(&qb[ks], &v, 16);
    }
  }
  // tiles: chunk c = tid + 256 u is key c / (D / 8), dims (c % (D / 8)) * 8 .. + 8; keys past
  // the prefix read zeros
  const int span = ((a.L - 1) * a.ts + D) * 2;
  const auto rk = make_rsrc(a.K + (size_t)g * a.hs, span);
  const auto rv = make_rsrc(a.V + (size_t)g * a.hs, span);
  uint4 pk[CPT], pv[CPT];   // the next tile to stage
  // K chunk c: key c / (D / 8), dims (c % (D / 8)) * 8 .. + 8 (16 lanes read one key's row);
  // V chunk c: key c % 32, dims (c / 32) * 8 .. + 8, so that the transposed 2-byte writes of
  // a wave's 32 lanes land on 32 consecutive keys of one dim row (16 banks) instead of 16
  // dim rows of one key.
  auto fetch = [&](int k0) {   // k0 past the prefix: zeros
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + NTH * u;
      const int kk = c / (D / 8), dc = c % (D / 8), vk = c % kPT, vd = c / kPT;
      pk[u] = load16(rk, c < CH ? ((k0 + kk) * a.ts + dc * 8) * 2 : span);
      pv[u] = load16(rv, c < CH ? ((k0 + vk) * a.ts + vd * 8) * 2 : span);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + NTH * u;
      const int kk = c / (D / 8), dc = c % (D / 8), vk = c % kPT, vd = c / kPT;
      if (c < CH) {
        *reinterpret_cast<uint4*>(sK[buf] + kk * KP + dc * 8) = pk[u];
        const uint16_t* e = reinterpret_cast<const uint16_t*>(&pv[u]);
#pragma unroll
        for (int i = 0; i < 8; ++i) sV[buf][(vd * 8 + i) * VP + vk] = e[i];
      }
    }
  };

  float m = -INFINITY, l = 0.f;   // per query column (both half-waves hold the same)
  f32x16_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[nt][j] = 0.f;

  const int ntile = (a.L + kPT - 1) / kPT;
  fetch(0);
  stage(0);
  fetch(kPT);
  __syncthreads();
  for (int t = 0; t < ntile; ++t) {
    const int cur = t & 1;
    // tile t + 1 into the other buffer (free since the last barrier), tile t + 2 into the
    // registers
    if (t + 1 < ntile) {
      stage(cur ^ 1);
      if (t + 2 < ntile) fetch((t + 2) * kPT);
    }
    if (active) {
      f32x16_t s;
#pragma unroll
      for (int j = 0; j < 16; ++j) s[j] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t A = *reinterpret_cast<const bf16x8_t*>(sK[cur] + col * KP + ks * 16 + half * 8);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qb[ks], s, 0, 0, 0);
      }
      // key of accumulator row j: 8 (j / 4) + 4 half + j % 4
      float p[16], mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = t * kPT + 8 * (j / 4) + 4 * half + (j & 3);
        p[j] = key < a.L ? s[j] * a.sl2 : -INFINITY;
        mx = fmaxf(mx, p[j]);
      }
      mx = fmaxf(mx, shfl_xor32(mx));
      // Lazy rescaling: the running max m moves only when a tile's max exceeds it by more
      // than 8 (log2 units), so every probability stays below 2^8 and the accumulators are
      // rescaled on few tiles; a / l is the same for any such m.  The first tile always moves
      // it (m = -inf; every tile holds a key of the prefix, so mx is finite).
      const float mn = mx > m + 8.f ? mx : m;
      const float corr = __builtin_amdgcn_exp2f(m - mn);   // 1 unless m moved
      float ls = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        p[j] = __builtin_amdgcn_exp2f(p[j] - mn);
        ls += p[j];
      }
      ls += shfl_xor32(ls);
      l = fmaf(l, corr, ls);
      m = mn;
      if (__builtin_amdgcn_ballot_w64(corr != 1.f)) {   // wave-uniform
        // the output rows are queries: their factors come through LDS (in order within a wave)
        if (half == 0) sRow[wave][col] = corr;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float cr = sRow[wave][8 * (j / 4) + 4 * half + (j & 3)];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[nt][j] *= cr;
        }
      }
      // P V: K-step kk takes this lane's p[8 kk .. 8 kk + 7], keys 16 kk + 8 (i / 4) + 4 half + i % 4
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float pp[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pp[i] = p[8 * kk + i];
        bf16x8_t ph, pm, plo;
        split3_bf16x8(pp, ph, pm, plo);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint16_t* vr = sV[cur] + (nt * 32 + col) * VP + 16 * kk + 4 * half;
          const uint2 v0 = *reinterpret_cast<const uint2*>(vr), v1 = *reinterpret_cast<const uint2*>(vr + 8);
          const uint4 bv = make_uint4(v0.x, v0.y, v1.x, v1.y);
          bf16x8_t B;
          __builtin_memcpy(&B, &bv, 16);
          acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph, B, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pm, B, acc[nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  if (!active) return;
  const float lse_c = (m + __builtin_amdgcn_logf(l)) * 0.6931471805599453f;   // this chunk's
  if (half == 0) {
    sRow[wave][col] = 1.f / l;
    sLse[wave][col] = lse_c;
  }
  // a later chunk merges with the state in memory by the online-softmax identity:
  // lse = log(e^lse_old + e^lse_c), a = e^(lse_old - lse) a_old + e^(lse_c - lse) a_c
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 8 * (j / 4) + 4 * half + (j & 3);
      if (q0 + r < a.N) {
        float* ap = a.a + ((size_t)(q0 + r) * a.H_q + h) * D + nt * 32 + col;
        float v = acc[nt][j] * sRow[wave][r];
        if (a.acc) {
          const float lo = a.lse[(size_t)(q0 + r) * a.H_q + h], lc = sLse[wave][r];
          const float mx = fmaxf(lo, lc);
          const float wo = __expf(lo - mx), wc = __expf(lc - mx);
          v = (wo * *ap + wc * v) / (wo + wc);
        }
        *ap = v;
      }
    }
  if (half == 0 && q0 + col < a.N) {
    float* lp = a.lse + (size_t)(q0 + col) * a.H_q + h;
    float out = lse_c;
    if (a.acc) {
      const float lo = *lp, mx = fmaxf(lo, lse_c);
      out = mx + __logf(__expf(lo - mx) + __expf(lse_c - mx));
    }
    *lp = out;
  }
}

// ------------------------------------------------------------------ K-means
// The centroids live in fp32 (C) and, for the matrix cores, as three bf16 planes
// (hi + mid + lo, ~24 bits) beside their squared norms; score(x, c) = ||c||^2 - 2 x . c
// orders a query's centroids as its squared distances do.
struct KmArgs {
  const uint16_t* X;   // [N, H, D] bf16
  float* C;            // [H, K, D]
  uint16_t* Cs;        // [H, 3, Kp, D] (Kp = K rounded up to 32; padding rows zero)
  float* cn2;          // [H, Kp] (padding rows +inf)
  int32_t* idx;        // [H, N]
  float* part;         // [H, nchunk, Kp, D + kRowExtra]: partial sums, count
  int N, H, K, Kp, rows;
};

constexpr int kRowExtra = 4;   // per partial row: D values, then the count (or Z), max lse, count

// A 32-centroid tile in LDS (fp32, rows past K zero) -> C (optionally), the split planes and
// the squared norms, each norm summed over the dims in order.
template <int D>
__device__ void write_centroid_tile(const KmArgs& a, int hh, int k0, float (*sC)[D + 4], bool write_c) {
  uint16_t* cs = a.Cs + (size_t)hh * 3 * a.Kp * D;
  for (int i = threadIdx.x; i < 32 * D; i += blockDim.x) {
    const int kk = i / D, c = i % D, k = k0 + kk;
    const float x = sC[kk][c];
    if (write_c && k < a.K) a.C[((size_t)hh * a.K + k) * D + c] = x;
    const __bf16 h = (__bf16)x;
    const float r1 = x - (float)h;
    const __bf16 m = (__bf16)r1;
    const __bf16 l = (__bf16)(r1 - (float)m);
    __builtin_memcpy(cs + (size_t)k * D + c, &h, 2);
    __builtin_memcpy(cs + ((size_t)a.Kp + k) * D + c, &m, 2);
    __builtin_memcpy(cs + ((size_t)2 * a.Kp + k) * D + c, &l, 2);
  }
  if (threadIdx.x < 32) {
    const int k = k0 + threadIdx.x;
    float s = 0.f;
    for (int c = 0; c < D; ++c) s = fmaf(sC[threadIdx.x][c], sC[threadIdx.x][c], s);
    a.cn2[(size_t)hh * a.Kp + k] = k < a.K ? s : INFINITY;
  }
}

// grid (Kp / 32, H), 256 threads: the initial centroids' planes and norms.
template <int D>
__global__ __launch_bounds__(256) void kmeans_prep_kernel(KmArgs a) {
  __shared__ float sC[32][D + 4];
  const int k0 = blockIdx.x * 32, hh = blockIdx.y;
  for (int i = threadIdx.x; i < 32 * D; i += 256) {
    const int kk = i / D, c = i % D;
    sC[kk][c] = k0 + kk < a.K ? a.C[((size_t)hh * a.K + k0 + kk) * D + c] : 0.f;
  }
  __syncthreads();
  write_centroid_tile<D>(a, hh, k0, sC, false);
}

// grid (ceil(N / 128), H), 256 threads: wave w scores queries 128 x + 32 w .. + 31 against
// 32-centroid tiles, S^T = C' X^T (centroids as rows), so each lane holds 16 centroids of
// one query; the lower score wins, ties keep the lower index.  The centroid tiles (three
// planes of 32 rows) come by direct buffer-to-LDS loads into a three-slot ring shared by the
// block's waves (rows of P 16-byte pieces, swizzled by piece_swz); a wave waits for its own
// loads of tile t before the block barrier while tiles t + 1 and t + 2 stay in flight.  (With
// every wave loading each tile itself, 16 bytes per lane over 32 rows and one tile at a
// time, an assignment pass over 4096 queries x 32 heads took ~98 us.)
template <int D>
__global__ __launch_bounds__(256) void kmeans_assign_kernel(KmArgs a) {
  constexpr int KS = D / 16;
  constexpr int P = D / 8;                    // 16-byte pieces per centroid row
  constexpr int NI = 3 * 32 * P / 64 / 4;     // 1 KB loads per wave per tile
  struct CTile { uint32_t w[3 * 32 * D / 2]; };   // [plane][32 rows][P pieces]
  __shared__ __attribute__((aligned(16))) CTile sC0, sC1, sC2;
  __shared__ float s_n2[256];
  const int hh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int q0 = blockIdx.x * 128 + wave * 32;
  bf16x8_t xb[KS];
  {
    const auto rx = make_rsrc(a.X + (size_t)hh * D, ((a.N - 1) * a.H * D + D) * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = load16(rx, ((q0 + col) * a.H * D + ks * 16 + half * 8) * 2);
      __builtin_memcpy(&xb[ks], &v, 16);
    }
  }
  for (int i = tid; i < a.Kp; i += 256) s_n2[i] = a.cn2[(size_t)hh * a.Kp + i];
  const auto rC = make_rsrc(a.Cs + (size_t)hh * 3 * a.Kp * D, 3 * a.Kp * D * 2);
  const int ntile = a.Kp / 32;
  auto issue = [&](int st, int t) {
    CTile* sc = st == 0 ? &sC0 : st == 1 ? &sC1 : &sC2;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int i = NI * wave + j;
      const int sl = i * 64 + lane, pl = sl / (32 * P), r = (sl / P) % 32, q = sl % P;
      const int off = ((pl * a.Kp + t * 32 + r) * D + 8 * (q ^ piece_swz<P>(r))) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rC, (__attribute__((address_space(3))) void*)(&sc->w[i * 256]), 16, off, 0, 0, 0);
    }
  };
  float best = INFINITY;
  int bi = 0;
  auto compute = [&](int st, int t) {
    const CTile* sc = st == 0 ? &sC0 : st == 1 ? &sC1 : &sC2;
    const int k0 = t * 32;
    f32x16_t acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // A operands: centroid row k0 + col, dims ks*16 + half*8 .. +8 of each plane
      const int pw = (col * P + ((2 * ks + half) ^ piece_swz<P>(col))) * 4;
      const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(&sc->w[pw]);
      const bf16x8_t am = *reinterpret_cast<const bf16x8_t*>(&sc->w[pw + 32 * P * 4]);
      const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(&sc->w[pw + 64 * P * 4]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xb[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, xb[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xb[ks], acc, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {   // centroid of row j: k0 + 8 (j / 4) + 4 half + j % 4 (increasing)
      const int k = k0 + 8 * (j / 4) + 4 * half + (j & 3);
      const float sc2 = fmaf(-2.f, acc[j], s_n2[k]);
      if (sc2 < best) { best = sc2; bi = k; }
    }
    // the tile's result is final here (left free, the compiler defers the comparisons of
    // several tiles past the next barriers and keeps their accumulators live)
    asm volatile("" : "+v"(best), "+v"(bi));
  };
  // step t: this wave's loads of tile t are done once at most those of tile t + 1 (NI) are
  // out; the barrier then also tells that every wave has finished with tile t - 1, whose slot
  // tile t + 2 takes (past the last tile the last one is loaded again, into a free slot)
  auto step = [&](int st, int t) {
    if constexpr (NI == 6) asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(3)\n\ts_barrier" ::: "memory");
    issue((st + 2) % 3, min(t + 2, ntile - 1));
    compute(st, t);
  };
  issue(0, 0);
  issue(1, min(1, ntile - 1));
  __syncthreads();   // the norms in LDS (and the first tiles landed)
  int t = 0;
  for (; t + 3 <= ntile; t += 3) {
    step(0, t);
    step(1, t + 1);
    step(2, t + 2);
  }
  if (t < ntile) step(0, t);
  if (t + 1 < ntile) step(1, t + 1);
  const float ob = shfl_xor32(best);
  const int oi = __shfl_xor(bi, 32);
  if (ob < best || (ob == best && oi < bi)) { best = ob; bi = oi; }
  if (half == 0 && q0 + col < a.N) a.idx[(size_t)hh * a.N + q0 + col] = bi;
}

// grid (nchunk, H), 512 threads: the partial sums of every centroid over one chunk of
// queries as one-hot contractions on the matrix cores: wave w owns centroids 32 w .. 32 w + 31
// (the one-hot A rows, from the assignment) and all D / 32 dim tiles (B = X^T of a 64-query
// stage in LDS).  The products are exact; the counts come from the same comparisons.
template <int D>
__global__ __launch_bounds__(512) void kmeans_part_kernel(KmArgs a) {
  constexpr int NT = D / 32, RS = 64, XP = RS + 8;
  constexpr int CPT = (RS * D / 8 + 511) / 512;   // 16-byte chunks per thread and stage
  __shared__ __align__(16) uint16_t sXT[D * XP];
  __shared__ int sIdx[RS];
  const int ch = blockIdx.x, hh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int kc = wave * 32 + col;   // this lane's centroid (one-hot row)
  const bool on = wave * 32 < a.Kp;
  f32x16_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[nt][j] = 0.f;
  int cnt = 0;
  const int r0 = ch * a.rows, r1 = min(a.N, r0 + a.rows);
  const auto rx = make_rsrc(a.X + (size_t)hh * D, ((a.N - 1) * a.H * D + D) * 2);
  const int32_t* ix = a.idx + (size_t)hh * a.N;
  uint4 px[CPT];
  int pid = -1;
  auto fetch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + 512 * u, rr = c / (D / 8), dc = c % (D / 8);
      const int r = s0 + rr;
      px[u] = load16(rx, (r < r1 && c < RS * D / 8) ? (r * a.H * D + dc * 8) * 2 : 0x7ffffff0);
    }
    pid = (tid < RS && s0 + tid < r1) ? ix[s0 + tid] : -1;
  };
  fetch(r0);
  for (int s0 = r0; s0 < r1; s0 += RS) {
    __syncthreads();   // the previous stage is consumed
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + 512 * u, rr = c / (D / 8), dc = c % (D / 8);
      if (c < RS * D / 8) {
        const uint16_t* e = reinterpret_cast<const uint16_t*>(&px[u]);
#pragma unroll
        for (int t = 0; t < 8; ++t) sXT[(dc * 8 + t) * XP + rr] = e[t];
      }
    }
    if (tid < RS) sIdx[tid] = pid;
    __syncthreads();
    if (s0 + RS < r1) fetch(s0 + RS);
    if (on) {
#pragma unroll
      for (int st = 0; st < RS / 16; ++st) {
        uint16_t oh[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool hit = sIdx[16 * st + 8 * half + e] == kc;
          oh[e] = hit ? 0x3F80 : 0;   // bf16 1.0
          cnt += hit;
        }
        bf16x8_t A;
        __builtin_memcpy(&A, oh, 16);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bf16x8_t B = *reinterpret_cast<const bf16x8_t*>(sXT + (nt * 32 + col) * XP + 16 * st + 8 * half);
          acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[nt], 0, 0, 0);
        }
      }
    }
  }
  if (!on) return;
  cnt += __shfl_xor(cnt, 32);
  constexpr int RW = D + kRowExtra;
  float* out = a.part + ((size_t)hh * gridDim.x + ch) * a.Kp * RW;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int k = wave * 32 + 8 * (j / 4) + 4 * half + (j & 3);
      out[(size_t)k * RW + nt * 32 + col] = acc[nt][j];
    }
  if (half == 0) out[(size_t)kc * RW + D] = (float)cnt;
}

// grid (Kp / 32, H), 256 threads: chunk partials summed in chunk order; a centroid with
// members becomes their mean, one without stays; then its planes and norm.
template <int D>
__global__ __launch_bounds__(256) void kmeans_reduce_kernel(KmArgs a, int nchunk) {
  constexpr int RW = D + kRowExtra;
  __shared__ float sC[32][D + 4];
  const int k0 = blockIdx.x * 32, hh = blockIdx.y;
  // thread: four consecutive dims of a centroid (16-byte loads of each chunk's partial row),
  // each summed over the chunks in chunk order
  static_assert(RW % 4 == 0, "16-byte aligned partial rows");
  for (int i = threadIdx.x; i < 32 * D / 4; i += 256) {
    const int kk = i / (D / 4), c = (i % (D / 4)) * 4, k = k0 + kk;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    float n = 0.f;
    for (int chn = 0; chn < nchunk; ++chn) {
      const float* p = a.part + (((size_t)hh * nchunk + chn) * a.Kp + k) * RW;
      const float4 v = *reinterpret_cast<const float4*>(p + c);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
      n += p[D];
    }
    const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = 0.f;
      if (k < a.K) v = n > 0.f ? sv[e] / n : a.C[((size_t)hh * a.K + k) * D + c + e];
      sC[kk][c + e] = v;
    }
  }
  __syncthreads();
  write_centroid_tile<D>(a, hh, k0, sC, true);
}

// ------------------------------------------------------------------ cluster states
// Every cluster's running online-softmax state of its members' (a, lse).
struct ClusterArgs {
  const float* A;       // [N, H, D] f32
  const float* lse;     // [N, H]
  const int32_t* idx;   // [H, N]
  float* part;          // [H, nchunk, K, D + kRowExtra]: e^(lse - max) weighted a, Z, max lse, count
  int N, H, K, rows;    // rows per chunk
};

// grid (nchunk, H), D threads: thread = one dim; the chunk's rows in index order, each folded
// into its cluster's LDS row (fixed order: deterministic).  Operands are fetched 8 rows ahead.
template <int D>
__global__ __launch_bounds__(D) void state_part_kernel(ClusterArgs a) {
  extern __shared__ float sAcc[];   // [K][D + kRowExtra]
  constexpr int RW = D + kRowExtra;
  const int ch = blockIdx.x, hh = blockIdx.y, tid = threadIdx.x;
  for (int i = tid; i < a.K * RW; i += D) sAcc[i] = i % RW == D + 1 ? -INFINITY : 0.f;
  __syncthreads();
  const int r0 = ch * a.rows, r1 = min(a.N, r0 + a.rows);
  const int32_t* ix = a.idx + (size_t)hh * a.N;
  for (int b0 = r0; b0 < r1; b0 += 8) {
    int k[8];
    float v[8], ls[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = min(b0 + u, r1 - 1);
      k[u] = ix[r];
      v[u] = a.A[((size_t)r * a.H + hh) * D + tid];
      ls[u] = a.lse[(size_t)r * a.H + hh];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (b0 + u >= r1) break;
      if (k[u] < 0 || k[u] >= a.K) continue;   // an assignment outside [0, K) joins no cluster
      float* acc = sAcc + k[u] * RW;
      // acc[D + 1] = max lse, acc[D] = sum e^(lse - max), acc[dim] = sum e^(lse - max) a
      const float mo = acc[D + 1], mn = fmaxf(mo, ls[u]);
      const float f = __expf(mo - mn), w = __expf(ls[u] - mn);
      acc[tid] = fmaf(acc[tid], f, w * v[u]);
      __syncthreads();   // every dim has read the old max
      if (tid == 0) { acc[D] = fmaf(acc[D], f, w); acc[D + 1] = mn; acc[D + 2] += 1.f; }
      __syncthreads();
    }
  }
  __syncthreads();
  float* out = a.part + ((size_t)hh * gridDim.x + ch) * a.K * RW;
  for (int i = tid; i < a.K * RW; i += D) out[i] = sAcc[i];
}

// grid (K, H), D threads: chunk states merged in chunk order:
// a_bar = sum_c e^(m_c - m) S_c / sum_c e^(m_c - m) Z_c, lse_bar = m + log Z - log n
// (a cluster without members: a_bar = 0, lse_bar = -inf).
template <int D>
__global__ __launch_bounds__(D) void state_reduce_kernel(const float* part, int nchunk, int K, float* a_bar,
                                                        float* lse_bar) {
  constexpr int RW = D + kRowExtra;
  const int k = blockIdx.x, hh = blockIdx.y, tid = threadIdx.x;
  const float* p0 = part + ((size_t)hh * nchunk * K + k) * RW;
  const size_t cs = (size_t)K * RW;   // chunk stride
  float m = -INFINITY, z = 0.f, s = 0.f, n = 0.f;
  for (int c = 0; c < nchunk; ++c) {
    const float mc = p0[c * cs + D + 1];
    if (mc == -INFINITY) continue;
    const float mn = fmaxf(m, mc);
    const float f = __expf(m - mn), fc = __expf(mc - mn);
    s = fmaf(s, f, fc * p0[c * cs + tid]);
    z = fmaf(z, f, fc * p0[c * cs + D]);
    n += p0[c * cs + D + 2];
    m = mn;
  }
  a_bar[((size_t)hh * K + k) * D + tid] = z > 0.f ? s / z : 0.f;
  if (tid == 0) lse_bar[(size_t)hh * K + k] = z > 0.f ? m + __logf(z) - __logf(n) : -INFINITY;
}

// ------------------------------------------------------------------ lookup + merge
// grid (H, b), 256 threads: cosine similarity of the query against the head's K centroids
// (q . c / ||c||; ||q|| does not change the argmax), the largest (ties: the lower index),
// then the retrieved state merged with the local one:
//   lse = log(e^lse_loc + e^lse_bar), o = e^(lse_loc - lse) o_loc + e^(lse_bar - lse) a_bar.
template <int D>
__global__ __launch_bounds__(256) void lookup_merge_kernel(const uint16_t* q, const float* C,
                                                          const float* a_bar, const float* lse_bar,
                                                          const float* o_loc, const float* lse_loc, float* o,
                                                          float* lse_out, int32_t* idx_out, int H, int K) {
  const int hh = blockIdx.x, bb = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float sq[D];
  __shared__ float s_best[4];
  __shared__ int s_bi[4];
  const size_t row = (size_t)bb * H + hh;
  if (tid < D) sq[tid] = bf16_to_f32(q[row * D + tid]);
  __syncthreads();
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int k = tid; k < K; k += 256) {
    const float* c = C + ((size_t)hh * K + k) * D;
    float dot = 0.f, n2 = 0.f;
#pragma unroll 8
    for (int i = 0; i < D; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(c + i);
      dot = fmaf(v.x, sq[i], dot);
      dot = fmaf(v.y, sq[i + 1], dot);
      dot = fmaf(v.z, sq[i + 2], dot);
      dot = fmaf(v.w, sq[i + 3], dot);
      n2 = fmaf(v.x, v.x, n2);
      n2 = fmaf(v.y, v.y, n2);
      n2 = fmaf(v.z, v.z, n2);
      n2 = fmaf(v.w, v.w, n2);
    }
    const float cs = n2 > 0.f ? dot * rsqrtf(n2) : -INFINITY;   // a centroid at the origin is never retrieved
    if (cs > best) { best = cs; bi = k; }
  }
  for (int off = 1; off < 64; off <<= 1) {
    const float ob = __shfl_xor(best, off);
    const int oi = __shfl_xor(bi, off);
    if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
  }
  if (lane == 0) { s_best[wave] = best; s_bi[wave] = bi; }
  __syncthreads();
  float b = s_best[0];
  int k = s_bi[0];
  for (int w = 1; w < 4; ++w)
    if (s_best[w] > b || (s_best[w] == b && s_bi[w] < k)) { b = s_best[w]; k = s_bi[w]; }
  if (k >= K) k = 0;   // every centroid at the origin: the first one (its state merges as is)
  const float l1 = lse_loc[row], l2 = lse_bar[(size_t)hh * K + k];
  const float mx = fmaxf(l1, l2);
  const float w1 = l1 == -INFINITY ? 0.f : __expf(l1 - mx), w2 = l2 == -INFINITY ? 0.f : __expf(l2 - mx);
  const float z = w1 + w2;
  if (tid < D) {
    const float v = z > 0.f ? (w1 * o_loc[row * D + tid] + w2 * a_bar[((size_t)hh * K + k) * D + tid]) / z : 0.f;
    o[row * D + tid] = v;
  }
  if (tid == 0) {
    idx_out[row] = k;
    if (lse_out) lse_out[row] = z > 0.f ? mx + __logf(z) : -INFINITY;
  }
}

}  // namespace kvm

using namespace kvm;

// ------------------------------------------------------------------ host side

static kvm_status check_asm_desc(const kvm_asm_desc* d) {
  KVM_PTR(d);
  KVM_REQUIRE(d->N > 0 && d->H_q > 0 && d->H_kv > 0 && d->L > 0, KVM_ERR_SHAPE, "N, H_q, H_kv, L must be positive");
  KVM_REQUIRE(d->d == 64 || d->d == 128, KVM_ERR_SHAPE, "head dim %d not in {64, 128}", d->d);
  KVM_REQUIRE(d->H_q % d->H_kv == 0, KVM_ERR_SHAPE, "H_q %d not a multiple of H_kv %d", d->H_q, d->H_kv);
  KVM_REQUIRE(d->dtype == KVM_BF16, KVM_ERR_DTYPE, "ASM takes bf16 queries and prefix (dtype %d)", d->dtype);
  KVM_REQUIRE(d->K >= 1 && d->K <= 256, KVM_ERR_RANGE, "K %d not in [1, 256]", d->K);
  // buffer offsets are 32-bit, and past-the-end offsets (reading zeros) must stay out of range
  KVM_REQUIRE((long long)d->N * d->H_q * d->d * 2 < 0x70000000LL, KVM_ERR_RANGE, "N x H_q x d too large");
  const long long ts = d->kv_head_major ? d->d : (long long)d->H_kv * d->d;
  KVM_REQUIRE(((long long)d->L * ts + d->d) * 2 < 0x70000000LL, KVM_ERR_RANGE, "prefix of %d tokens too long", d->L);
  return KVM_OK;
}

static int asm_chunk_rows(const kvm_asm_desc* d) { return 512; }
static int asm_chunks(const kvm_asm_desc* d) { return (d->N + asm_chunk_rows(d) - 1) / asm_chunk_rows(d); }

struct AsmWs { size_t cs, cn2, part, total; };
static int asm_kp(const kvm_asm_desc* d) { return (d->K + 31) / 32 * 32; }
static AsmWs asm_ws(const kvm_asm_desc* d) {
  const size_t H = d->H_q, Kp = asm_kp(d);
  AsmWs w;
  w.cs = 0;
  w.cn2 = align_up(H * 3 * Kp * d->d * sizeof(uint16_t), 256);
  w.part = align_up(w.cn2 + H * Kp * sizeof(float), 256);
  w.total = align_up(w.part + H * asm_chunks(d) * Kp * (d->d + kRowExtra) * sizeof(float), 256);
  return w;
}

static kvm_status set_lds(const void* fn, int bytes) {
  if (bytes <= 65536) return KVM_OK;
  return check_hip(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes), "LDS size");
}

extern "C" size_t kvm_asm_workspace_size(const kvm_asm_desc* d) {
  if (check_asm_desc(d) != KVM_OK) return 0;
  return asm_ws(d).total;
}

extern "C" kvm_status kvm_asm_prefix_states(const kvm_asm_desc* d, const void* Q, const void* K, const void* V,
                                            float* a_out, float* lse_out, int32_t accumulate, void* stream) {
  kvm_status st = check_asm_desc(d);
  if (st != KVM_OK) return st;
  KVM_PTR_ALIGNED(Q); KVM_PTR_ALIGNED(K); KVM_PTR_ALIGNED(V); KVM_PTR_ALIGNED(a_out); KVM_PTR_ALIGNED(lse_out);
  st = require_gfx950();
  if (st != KVM_OK) return st;
  PrefixArgs a{};
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.a = a_out; a.lse = lse_out; a.acc = accumulate != 0;
  a.N = d->N; a.H_q = d->H_q; a.G = d->H_q / d->H_kv; a.L = d->L;
  a.ts = d->kv_head_major ? d->d : d->H_kv * d->d;
  a.hs = d->kv_head_major ? d->L * d->d : d->d;
  a.sl2 = 1.4426950408889634f / sqrtf((float)d->d);
  const int items = a.G * ((d->N + 31) / 32);
  const dim3 grid((items + kPW - 1) / kPW, d->H_kv);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->d == 128) hipLaunchKernelGGL(prefix_states_kernel<128>, grid, dim3(64 * kPW), 0, s, a);
  else hipLaunchKernelGGL(prefix_states_kernel<64>, grid, dim3(64 * kPW), 0, s, a);
  return check_hip(hipGetLastError(), "prefix states launch");
}

template <int D>
static void kmeans_run(const KmArgs& a, int iters, int nchunk, hipStream_t s) {
  const dim3 tgrid(a.Kp / 32, a.H), agrid((a.N + 127) / 128, a.H), pgrid(nchunk, a.H);
  hipLaunchKernelGGL(kmeans_prep_kernel<D>, tgrid, dim3(256), 0, s, a);
  for (int it = 0; it <= iters; ++it) {
    hipLaunchKernelGGL(kmeans_assign_kernel<D>, agrid, dim3(256), 0, s, a);
    if (it == iters) break;
    hipLaunchKernelGGL(kmeans_part_kernel<D>, pgrid, dim3(512), 0, s, a);
    hipLaunchKernelGGL(kmeans_reduce_kernel<D>, tgrid, dim3(256), 0, s, a, nchunk);
  }
}

extern "C" kvm_status kvm_asm_kmeans(const kvm_asm_desc* d, const void* Q, float* C, int32_t* idx, int32_t iters,
                                     void* ws, size_t ws_bytes, void* stream) {
  kvm_status st = check_asm_desc(d);
  if (st != KVM_OK) return st;
  KVM_REQUIRE(iters >= 0, KVM_ERR_RANGE, "iters %d < 0", iters);
  KVM_PTR_ALIGNED(Q); KVM_PTR_ALIGNED(C); KVM_PTR_ALIGNED(idx);
  const AsmWs w = asm_ws(d);
  KVM_REQUIRE(ws != nullptr && ws_bytes >= w.total, KVM_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  KVM_ALIGNED(ws);
  st = require_gfx950();
  if (st != KVM_OK) return st;
  char* base = static_cast<char*>(ws);
  KmArgs a{};
  a.X = static_cast<const uint16_t*>(Q);
  a.C = C;
  a.Cs = reinterpret_cast<uint16_t*>(base + w.cs);
  a.cn2 = reinterpret_cast<float*>(base + w.cn2);
  a.idx = idx;
  a.part = reinterpret_cast<float*>(base + w.part);
  a.N = d->N; a.H = d->H_q; a.K = d->K; a.Kp = asm_kp(d); a.rows = asm_chunk_rows(d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->d == 128) kmeans_run<128>(a, iters, asm_chunks(d), s);
  else kmeans_run<64>(a, iters, asm_chunks(d), s);
  return check_hip(hipGetLastError(), "kmeans launch");
}

extern "C" kvm_status kvm_asm_cluster_states(const kvm_asm_desc* d, const float* a_in, const float* lse_in,
                                             const int32_t* idx, float* a_bar, float* lse_bar, void* ws,
                                             size_t ws_bytes, void* stream) {
  kvm_status st = check_asm_desc(d);
  if (st != KVM_OK) return st;
  KVM_PTR_ALIGNED(a_in); KVM_PTR_ALIGNED(lse_in); KVM_PTR_ALIGNED(idx); KVM_PTR_ALIGNED(a_bar);
  KVM_PTR_ALIGNED(lse_bar);
  const AsmWs w = asm_ws(d);
  KVM_REQUIRE(ws != nullptr && ws_bytes >= w.total, KVM_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  KVM_ALIGNED(ws);
  st = require_gfx950();
  if (st != KVM_OK) return st;
  ClusterArgs ca{};
  ca.A = a_in; ca.lse = lse_in; ca.idx = idx; ca.part = reinterpret_cast<float*>(static_cast<char*>(ws) + w.part);
  ca.N = d->N; ca.H = d->H_q; ca.K = d->K; ca.rows = asm_chunk_rows(d);
  const int nchunk = asm_chunks(d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int lds = d->K * (d->d + kRowExtra) * (int)sizeof(float);
  if (d->d == 128) {
    st = set_lds(reinterpret_cast<const void*>(&state_part_kernel<128>), lds);
    if (st != KVM_OK) return st;
    hipLaunchKernelGGL(state_part_kernel<128>, dim3(nchunk, ca.H), dim3(128), lds, s, ca);
    hipLaunchKernelGGL(state_reduce_kernel<128>, dim3(ca.K, ca.H), dim3(128), 0, s, ca.part, nchunk, ca.K, a_bar,
                       lse_bar);
  } else {
    st = set_lds(reinterpret_cast<const void*>(&state_part_kernel<64>), lds);
    if (st != KVM_OK) return st;
    hipLaunchKernelGGL(state_part_kernel<64>, dim3(nchunk, ca.H), dim3(64), lds, s, ca);
    hipLaunchKernelGGL(state_reduce_kernel<64>, dim3(ca.K, ca.H), dim3(64), 0, s, ca.part, nchunk, ca.K, a_bar,
                       lse_bar);
  }
  return check_hip(hipGetLastError(), "cluster states launch");
}

extern "C" kvm_status kvm_asm_lookup(const kvm_asm_desc* d, int32_t b, const void* q, const float* C,
                                     const float* a_bar, const float* lse_bar, const float* o_loc,
                                     const float* lse_loc, float* o, float* lse_out, int32_t* idx_out,
                                     void* stream) {
  kvm_status st = check_asm_desc(d);
  if (st != KVM_OK) return st;
  KVM_REQUIRE(b > 0, KVM_ERR_SHAPE, "b must be positive");
  KVM_PTR_ALIGNED(q); KVM_PTR_ALIGNED(C); KVM_PTR_ALIGNED(a_bar); KVM_PTR_ALIGNED(lse_bar); KVM_PTR_ALIGNED(o_loc);
  KVM_PTR_ALIGNED(lse_loc); KVM_PTR_ALIGNED(o); KVM_PTR_ALIGNED(idx_out); KVM_OPT_ALIGNED(lse_out);
  st = require_gfx950();
  if (st != KVM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(d->H_q, b);
  const auto* qb = static_cast<const uint16_t*>(q);
  if (d->d == 128)
    hipLaunchKernelGGL(lookup_merge_kernel<128>, grid, dim3(256), 0, s, qb, C, a_bar, lse_bar, o_loc, lse_loc, o,
                       lse_out, idx_out, d->H_q, d->K);
  else
    hipLaunchKernelGGL(lookup_merge_kernel<64>, grid, dim3(256), 0, s, qb, C, a_bar, lse_bar, o_loc, lse_loc, o,
                       lse_out, idx_out, d->H_q, d->K);
  return check_hip(hipGetLastError(), "asm lookup launch");
}
