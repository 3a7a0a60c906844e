// V1 / V3: MomentKV's eviction score and its normalization-corrected read-out [MKV].
//
// alpha_j = (1 / (W G)) sum over the window's queries s and the G query heads of the KV
// group of the causal softmax weight of key j (the attention mass each key receives);
// score_j = alpha_j ||r_j||, r_j = v_j - v_bar - S~ k_j / (n_e sqrt d) (r_j = v_j while
// nothing is evicted) [MKV part 3]; the read-out mixes the retained attention output with
// the first-order estimate of the evicted one [MKV parts 2 and 4].
//
// alpha runs on the matrix cores in two passes over the same 32 x 32 logit tiles:
//   pass 1: C = K Q^T (keys as rows): each lane owns one query column and keeps an online
//           (max, sum) of exp2 over its key rows -> partial log-sum-exp per query and chunk;
//   merge:  log-sum-exp per query over the chunks;
//   pass 2: C = Q K^T (queries as rows): each lane owns one key column and sums
//           exp2(logit - lse) over its query rows -> alpha per key.
// Swapping the operands between the passes keeps every reduction inside a lane (plus one
// exchange between the two half-waves), so no cross-lane row reductions are needed.
#include "common.hpp"

namespace kvm {

struct AlphaArgs {
  const uint16_t* Q;   // [b, W, H_q, d]
  const uint16_t* K;
  float* alpha;        // [b, H_kv, L]
  float2* part;        // ws [pairs, chunks, WG]  (max, sum) in log2 units
  float* lse2;         // ws [pairs, WG]
  int L, H_q, H_kv, W, G, WG, n_chunks;
  long long tok_stride, head_stride, batch_stride;
  float scale_log2;    // scale * log2(e)
};

// Keys per block: 2048 where that still gives 512 blocks, else 512.  Every block loads its
// group's window queries, so longer chunks load them less often (32K tokens x batch 4: both
// passes 0.329 -> 0.281 ms).
static int alpha_chunk(int L, int pairs) { return (long long)((L + 2047) / 2048) * pairs >= 512 ? 2048 : 512; }
constexpr int kAlphaQPW = 2;       // 32-row query tiles per wave (W G <= 256)

template <int D, int PASS, int kAlphaChunk>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void moment_alpha_kernel(AlphaArgs a) {
  constexpr int KS = D / 16;
  const int c = blockIdx.x, pair = blockIdx.y;
  const int bb = pair / a.H_kv, g = pair % a.H_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  constexpr int P = D / 8;                    // 16-byte pieces per key row
  constexpr int NI = 32 * P / 64 / 4;         // 1 KB loads per wave per key tile
  struct KeyTile { uint32_t w[16 * D]; };
  __shared__ __attribute__((aligned(16))) KeyTile sK0, sK1, sK2;
  __shared__ float s_alpha[4][kAlphaChunk];

  // query operands of this wave's tiles: rows r = s G + hh of the group (q of position L-W+s)
  bf16x8_t qop[kAlphaQPW][KS];
#pragma unroll
  for (int x = 0; x < kAlphaQPW; ++x) {
    const int r = (wave * kAlphaQPW + x) * 32 + col;
    const bool ok = r < a.WG;
    const int s = ok ? r / a.G : 0, hh = ok ? r % a.G : 0;
    const uint16_t* qp = a.Q + (((size_t)bb * a.W + s) * a.H_q + g * a.G + hh) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ok) v = *reinterpret_cast<const uint4*>(qp + ks * 16);
      __builtin_memcpy(&qop[x][ks], &v, 16);
    }
  }
  // pass 2: log-sum-exp of the 16 query rows this lane holds per tile
  float lq[kAlphaQPW][16];
  if (PASS == 2) {
#pragma unroll
    for (int x = 0; x < kAlphaQPW; ++x)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = (wave * kAlphaQPW + x) * 32 + 8 * (j / 4) + 4 * half + (j % 4);
        lq[x][j] = r < a.WG ? a.lse2[(size_t)pair * a.WG + r] : INFINITY;
      }
  }
  float m[kAlphaQPW], l[kAlphaQPW];
#pragma unroll
  for (int x = 0; x < kAlphaQPW; ++x) { m[x] = -INFINITY; l[x] = 0.f; }

  const int k0 = c * kAlphaChunk;
  const int ntile = min(kAlphaChunk, a.L - k0 + 31) / 32;
  const int p0 = a.L - a.W;   // position of window query 0
  // Key tile t (32 rows) moves into LDS slot t % 3 by direct buffer-to-LDS loads, NI per
  // wave, each moving 1 KB (lane i writes the 16-byte piece i).  Piece q of row r holds dims
  // 8 (q ^ piece_swz<P>(r)) .. +8 of key r, so the operand reads (16 rows of one 16-byte column per
  // phase) meet no bank conflicts; rows past L read zeros.  A wave waits for its own loads
  // of tile t, then the block barrier makes every wave's pieces visible, while tiles t + 1
  // and t + 2 stay in flight: with one tile in flight per block (8 KB) the pass ran at the
  // rate its loads in flight allow (~2 TB/s).
  const int span = (int)(((long long)(a.L - 1) * a.tok_stride + D) * 2);
  const auto rK = make_rsrc(a.K + bb * a.batch_stride + g * a.head_stride, span);
  auto issue = [&](int st, int t) {
    KeyTile* sk = st == 0 ? &sK0 : st == 1 ? &sK1 : &sK2;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int i = NI * wave + j;
      const int sl = i * 64 + lane, r = sl / P, q = sl % P;
      const int off = ((k0 + t * 32 + r) * (int)a.tok_stride + 8 * (q ^ piece_swz<P>(r))) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (__attribute__((address_space(3))) void*)(&sk->w[i * 256]), 16, off, 0, 0, 0);
    }
  };
  auto compute = [&](int st, int t) {
    const KeyTile* sk = st == 0 ? &sK0 : st == 1 ? &sK1 : &sK2;
    const int kb = k0 + t * 32;
    // a tile whose keys every window query sees (and all below L) needs no causal mask
    const bool interior = kb + 31 <= p0;
    // key operand: key row `col`, k-slice half*8 .. +8 of each k-step
    bf16x8_t kop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = *reinterpret_cast<const uint4*>(&sk->w[(col * P + ((2 * ks + half) ^ piece_swz<P>(col))) * 4]);
      __builtin_memcpy(&kop[ks], &v, 16);
    }
    float asum = 0.f;
#pragma unroll
    for (int x = 0; x < kAlphaQPW; ++x) {
      f32x16_t acc;
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = PASS == 1 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[x][ks], acc, 0, 0, 0)
                        : __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[x][ks], kop[ks], acc, 0, 0, 0);
      const int rbase = (wave * kAlphaQPW + x) * 32;
      if (PASS == 1) {
        // rows = keys, this lane's column = query r
        const int r = rbase + col;
        const int lim = r < a.WG ? min(a.L - 1, p0 + r / a.G) : -1;   // last visible key
        float z[16], mt = -INFINITY;
        if (interior) {   // (rows past W G only fill state that is never written)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            z[j] = acc[j] * a.scale_log2;
            mt = fmaxf(mt, z[j]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = kb + 8 * (j / 4) + 4 * half + (j % 4);
            z[j] = key <= lim ? acc[j] * a.scale_log2 : -INFINITY;
            mt = fmaxf(mt, z[j]);
          }
        }
        // no branch on an empty column: with the maximum still -inf every term is 0 and the
        // state stays (-inf, 0)
        const float mn = fmaxf(m[x], mt);
        const float msafe = mn == -INFINITY ? 0.f : mn;
        float sacc = l[x] * __builtin_amdgcn_exp2f(m[x] - msafe);
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc += __builtin_amdgcn_exp2f(z[j] - msafe);
        l[x] = sacc;
        m[x] = mn;
      } else {
        // rows = queries, this lane's column = key kb + col
        const int key = kb + col;
        if (interior) {   // rows past W G: lq = inf, so their terms are +0
#pragma unroll
          for (int j = 0; j < 16; ++j) asum += __builtin_amdgcn_exp2f(acc[j] * a.scale_log2 - lq[x][j]);
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int r = rbase + 8 * (j / 4) + 4 * half + (j % 4);
            const bool vis = r < a.WG && key < a.L && key <= p0 + r / a.G;
            asum += vis ? __builtin_amdgcn_exp2f(acc[j] * a.scale_log2 - lq[x][j]) : 0.f;
          }
        }
      }
    }
    if (PASS == 2) {
      asum += shfl_xor32(asum);
      s_alpha[wave][t * 32 + col] = asum;   // both half-waves hold the same sum
    } else {
      // the tile's softmax state is final here: left free, the compiler defers the epilogues
      // of three tiles past the next barriers and keeps their accumulators live meanwhile
#pragma unroll
      for (int x = 0; x < kAlphaQPW; ++x) asm volatile("" : "+v"(m[x]), "+v"(l[x]));
    }
  };
  // step t: this wave's loads of tile t are done once at most those of tile t + 1 (NI) are
  // out; the barrier then also tells that every wave has finished with tile t - 1, whose slot
  // tile t + 2 takes (past the last tile the last one is loaded again, into a free slot)
  auto step = [&](int st, int t) {
    if constexpr (NI == 2) asm volatile("s_waitcnt vmcnt(2)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(1)\n\ts_barrier" ::: "memory");
    issue((st + 2) % 3, min(t + 2, ntile - 1));
    compute(st, t);
  };
  issue(0, 0);
  issue(1, min(1, ntile - 1));
  int t = 0;
  for (; t + 3 <= ntile; t += 3) {
    step(0, t);
    step(1, t + 1);
    step(2, t + 2);
  }
  if (t < ntile) step(0, t);
  if (t + 1 < ntile) step(1, t + 1);
  __syncthreads();
  if (PASS == 1) {
    // combine the two half-waves (same query column, different key rows)
#pragma unroll
    for (int x = 0; x < kAlphaQPW; ++x) {
      const float om = shfl_xor32(m[x]), ol = shfl_xor32(l[x]);
      const float mn = fmaxf(m[x], om);
      float sum = 0.f;
      if (mn != -INFINITY) sum = l[x] * __builtin_amdgcn_exp2f(m[x] - mn) + ol * __builtin_amdgcn_exp2f(om - mn);
      const int r = (wave * kAlphaQPW + x) * 32 + col;
      if (half == 0 && r < a.WG) a.part[((size_t)pair * a.n_chunks + c) * a.WG + r] = make_float2(mn, sum);
    }
  } else {
    const float inv = 1.f / (float)a.WG;
    for (int i = tid; i < ntile * 32; i += 256) {
      const int j = k0 + i;
      if (j < a.L) {
        const float s = ((s_alpha[0][i] + s_alpha[1][i]) + s_alpha[2][i]) + s_alpha[3][i];
        a.alpha[(size_t)pair * a.L + j] = s * inv;
      }
    }
  }
}

// grid (pairs), 256 threads: log-sum-exp (log2 units) of each query row over the chunks.
__global__ __launch_bounds__(256) void alpha_merge_kernel(AlphaArgs a) {
  const int pair = blockIdx.x;
  for (int r = threadIdx.x; r < a.WG; r += 256) {
    float mx = -INFINITY;
    for (int c = 0; c < a.n_chunks; ++c) mx = fmaxf(mx, a.part[((size_t)pair * a.n_chunks + c) * a.WG + r].x);
    float s = 0.f;
    if (mx != -INFINITY)
      for (int c = 0; c < a.n_chunks; ++c) {
        const float2 p = a.part[((size_t)pair * a.n_chunks + c) * a.WG + r];
        if (p.x != -INFINITY) s += p.y * __builtin_amdgcn_exp2f(p.x - mx);
      }
    a.lse2[(size_t)pair * a.WG + r] = mx + log2f(s);
  }
}

// ------------------------------------------------------------------ residual score
// grid (ceil(L / KEYS), pairs), D / 32 waves (KEYS = 256, or 1024 where the grid keeps a
// block per CU: each block splits its S once, so larger blocks repeat that less; 32K tokens
// x batch 4: 0.286 -> 0.251 ms).  The K and V tiles are shared by the block's waves through
// LDS (each byte fetched once per block, in whole cache lines): with every wave loading the
// whole K tile itself the round took 0.25 ms, with the shared tiles 0.11 ms.
// residual: C[i][key] = sum_c S'[i][c] k[key][c] with S' = S~ / (n_e sqrt d) split into
// three bf16 terms (hi + mid + lo, ~24 bits) as the A operand and the exact bf16 keys as
// the B operand; r = v - v_bar - C; ||r||^2 sums the lane's rows, the two half-waves and
// the waves.
struct ScoreArgs {
  const uint16_t* K;
  const uint16_t* V;
  const float* alpha;   // [pairs, L]
  const int32_t* n_e;
  const float* s_k;
  const float* s_v;
  const float* S;
  float* score;         // [pairs, L]
  int L, H_kv;
  long long tok_stride, head_stride, batch_stride;
  float inv_sqrt_d;
};


template <int D, int KEYS>
__global__ __launch_bounds__(D * 2) void moment_score_kernel(ScoreArgs a) {
  constexpr int kScoreKeys = KEYS;
  constexpr int KS = D / 16;
  constexpr int NW = D / 32;
  const int c = blockIdx.x, pair = blockIdx.y;
  const int bb = pair / a.H_kv, g = pair % a.H_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  // LDS K/V tiles: 32 rows of P 16-byte pieces, swizzled by piece_swz
  constexpr int P = D / 8;
  struct SharedTile { uint32_t w[16 * D]; };
  __shared__ __attribute__((aligned(16))) SharedTile s_k0, s_k1, s_k2, s_v0, s_v1, s_v2;
  __shared__ float s_ss[NW][kScoreKeys];

  const int ne = a.n_e[pair];
  const float inv_n = (ne > 0 ? 1.f : 0.f) / (float)max(ne, 1);   // no branch on the count
  const float* sk = a.s_k + (size_t)pair * D;
  const float* sv = a.s_v + (size_t)pair * D;
  // A operands: row i = 32 wave + col of S' (zero while nothing is evicted).  Every load is
  // unconditional; the count only selects the result, so no load waits behind a branch.
  const int i_row = wave * 32 + col;
  bf16x8_t sh[KS], sm[KS], sl[KS];
  {
    const float* Sr = a.S + ((size_t)pair * D + i_row) * D;
    const float svi = sv[i_row];
    const float f = inv_n * a.inv_sqrt_d;
    float4 s4[KS][2], k4[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        s4[ks][u] = *reinterpret_cast<const float4*>(Sr + ks * 16 + half * 8 + 4 * u);
        k4[ks][u] = *reinterpret_cast<const float4*>(sk + ks * 16 + half * 8 + 4 * u);
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float sr = e < 4 ? (&s4[ks][0].x)[e] : (&s4[ks][1].x)[e - 4];
        const float kv = e < 4 ? (&k4[ks][0].x)[e] : (&k4[ks][1].x)[e - 4];
        x[e] = ne > 0 ? (sr - svi * kv * inv_n) * f : 0.f;
      }
      split3_bf16x8(x, sh[ks], sm[ks], sl[ks]);
    }
  }
  // v_bar of the 16 dims this lane holds in the C layout
  float vbar[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) vbar[j] = sv[wave * 32 + 8 * (j / 4) + 4 * half + (j % 4)] * inv_n;

  // K and V of this (sequence, KV head) through buffer resources that end after token L-1:
  // keys past the end read zeros, so no load is conditional
  const int tb = (int)sizeof(uint16_t);
  const int span = (int)(((long long)(a.L - 1) * a.tok_stride + D) * tb);
  const auto rK = make_rsrc(a.K + bb * a.batch_stride + g * a.head_stride, span);
  const auto rV = make_rsrc(a.V + bb * a.batch_stride + g * a.head_stride, span);
  const int k0 = c * kScoreKeys;
  const int ntile = min(kScoreKeys, a.L - k0 + 31) / 32;
  // Tile t (32 keys) of K and of V moves into LDS slot t % 3 by direct buffer-to-LDS loads:
  // each of the 2 NW loads per tensor moves 1 KB, lane i writing the 16-byte piece i.  Piece
  // q of row r holds dims 8 (q ^ piece_swz<P>(r)) .. +8 of key r, so the MFMA operand reads (16 rows
  // of one 16-byte column per phase) meet no bank conflicts.  A wave waits for its own loads
  // of a tile, then the block barrier makes every wave's pieces visible; tiles t + 1 and
  // t + 2 stay in flight meanwhile.
  const auto kpiece = [&](int t, int i) {
    const int s = i * 64 + lane;                  // slot of this lane's piece
    const int r = s / P, q = s % P;
    const int key = k0 + t * 32 + r;
    return (key * (int)a.tok_stride + 8 * (q ^ piece_swz<P>(r))) * tb;
  };
  auto issue = [&](int st, int t) {
    SharedTile* sk = st == 0 ? &s_k0 : st == 1 ? &s_k1 : &s_k2;
    SharedTile* svv = st == 0 ? &s_v0 : st == 1 ? &s_v1 : &s_v2;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = 2 * wave + j;
      const int off = kpiece(t, i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (__attribute__((address_space(3))) void*)(&sk->w[i * 256]), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (__attribute__((address_space(3))) void*)(&svv->w[i * 256]), 16, off, 0, 0, 0);
    }
  };
  auto compute = [&](int st, int t) {
    const SharedTile* sk = st == 0 ? &s_k0 : st == 1 ? &s_k1 : &s_k2;
    const SharedTile* svv = st == 0 ? &s_v0 : st == 1 ? &s_v1 : &s_v2;
    uint2 vv[4];
    f32x16_t acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // B operand: key col, dims ks*16 + half*8 .. +8
      const uint4 kvv = *reinterpret_cast<const uint4*>(&sk->w[(col * P + ((2 * ks + half) ^ piece_swz<P>(col))) * 4]);
      bf16x8_t B;
      __builtin_memcpy(&B, &kvv, 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sh[ks], B, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sm[ks], B, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sl[ks], B, acc, 0, 0, 0);
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)    // dims wave*32 + 8 q4 + 4 half .. +4 of this key's v
      vv[q4] = *reinterpret_cast<const uint2*>(&svv->w[(col * P + ((wave * 4 + q4) ^ piece_swz<P>(col))) * 4 + half * 2]);
    float ss = 0.f;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      // rows 8 q4 + 4 half + 0..3 of the C tile
      const float v4[4] = {bf16_lo(vv[q4].x), bf16_hi(vv[q4].x), bf16_lo(vv[q4].y), bf16_hi(vv[q4].y)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float r = v4[e] - vbar[q4 * 4 + e] - acc[q4 * 4 + e];
        ss = fmaf(r, r, ss);
      }
    }
    ss += shfl_xor32(ss);
    s_ss[wave][t * 32 + col] = ss;   // both half-waves hold the same sum
  };
  // step t: this wave's loads of tile t are done once at most those of tile t + 1 (4) are
  // out; the barrier then also tells that every wave has finished with tile t - 1, whose slot
  // tile t + 2 takes (past the last tile the last one is loaded again, into a free slot)
  auto step = [&](int st, int t) {
    asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    issue((st + 2) % 3, min(t + 2, ntile - 1));
    compute(st, t);
  };
  issue(0, 0);
  issue(1, min(1, ntile - 1));
  int t = 0;
  for (; t + 3 <= ntile; t += 3) {
    step(0, t);
    step(1, t + 1);
    step(2, t + 2);
  }
  if (t < ntile) step(0, t);
  if (t + 1 < ntile) step(1, t + 1);
  __syncthreads();
  for (int i = tid; i < ntile * 32; i += NW * 64) {
    const int j = k0 + i;
    if (j < a.L) {
      float ss = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) ss += s_ss[w][i];
      a.score[(size_t)pair * a.L + j] = a.alpha[(size_t)pair * a.L + j] * sqrtf(ss);
    }
  }
}

// ------------------------------------------------------------------ read-out (V3)
// grid (H_kv, b), 256 threads.  Per query head h of the group:
//   f_E = v_bar + (S q - s_v (s_k . q) / n_e) / (n_e sqrt d),  log Z_E = log n_e + (q . s_k / n_e) / sqrt d,
//   w_R = sigmoid(lse_R - log Z_E),  o = w_R f_R + (1 - w_R) f_E   (o = f_R while n_e = 0).
template <typename T>
__global__ __launch_bounds__(256) void moment_readout_kernel(const T* q, const float* fR, const float* lseR,
                                                             const int32_t* n_e, const float* s_k, const float* s_v,
                                                             const float* S, float* o, int H_q, int H_kv, int D,
                                                             float scale) {
  const int g = blockIdx.x, bb = blockIdx.y, tid = threadIdx.x;
  const int G = H_q / H_kv;
  const size_t pair = (size_t)bb * H_kv + g;
  extern __shared__ float smem[];
  float* sq = smem;              // [G][D]
  float* sr = smem + G * D;      // [G]: s_k . q
  for (int i = tid; i < G * D; i += 256) sq[i] = load_scalar<T>(q + ((size_t)bb * H_q + g * G) * D + i);
  __syncthreads();
  const int ne = n_e[pair];
  const float* sk = s_k + pair * D;
  if (tid < 64) {
    for (int h = 0; h < G; ++h) {
      float x = 0.f;
      for (int i = tid; i < D; i += 64) x = fmaf(sk[i], sq[h * D + i], x);
      x = wave_sum(x);
      if (tid == 0) sr[h] = x;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, i = idx % D;
    const size_t oh = ((size_t)bb * H_q + g * G + h) * D + i;
    const float f = fR[oh];
    if (ne <= 0) { o[oh] = f; continue; }
    const float* Sr = S + (pair * D + i) * D;
    float sq_i = 0.f;
    for (int cc = 0; cc < D; ++cc) sq_i = fmaf(Sr[cc], sq[h * D + cc], sq_i);
    const float inv = 1.f / (float)ne;
    const float sv = s_v[pair * D + i];
    const float fE = sv * inv + scale * (sq_i - sv * sr[h] * inv) * inv;
    const float logZ = __logf((float)ne) + scale * sr[h] * inv;
    const float w = sigmoid_f(lseR[(size_t)bb * H_q + g * G + h] - logZ);
    o[oh] = w * f + (1.f - w) * fE;
  }
}

struct MomentWs { size_t part, lse, total; };
static MomentWs moment_ws(const kvm_moment_desc* d) {
  const size_t pairs = (size_t)d->b * d->H_kv;
  const int nc = (d->L + alpha_chunk(d->L, (int)pairs) - 1) / alpha_chunk(d->L, (int)pairs);
  const int WG = d->W * (d->H_q / d->H_kv);
  MomentWs w;
  w.part = 0;
  w.lse = align_up(pairs * nc * WG * sizeof(float2), 256);
  w.total = align_up(w.lse + pairs * WG * sizeof(float), 256);
  return w;
}

static void strides(const kvm_moment_desc* d, long long& ts, long long& hs, long long& bs) {
  if (d->kv_head_major) {
    ts = d->d; hs = (long long)d->L * d->d; bs = (long long)d->H_kv * d->L * d->d;
  } else {
    ts = (long long)d->H_kv * d->d; hs = d->d; bs = (long long)d->L * d->H_kv * d->d;
  }
}

static kvm_status check_moment_desc(const kvm_moment_desc* d) {
  KVM_PTR(d);
  KVM_REQUIRE(d->b > 0 && d->L > 0 && d->H_kv > 0, KVM_ERR_SHAPE, "b, L, H_kv must be positive");
  KVM_REQUIRE(d->d == 64 || d->d == 128, KVM_ERR_SHAPE, "head dim %d not in {64, 128}", d->d);
  KVM_REQUIRE(d->dtype == KVM_BF16, KVM_ERR_DTYPE, "MomentKV scoring takes bf16 K, V, Q (dtype %d)", d->dtype);
  return KVM_OK;
}

}  // namespace kvm

using namespace kvm;

extern "C" size_t kvm_moment_workspace_size(const kvm_moment_desc* d) {
  if (!d || d->b <= 0 || d->L <= 0 || d->H_kv <= 0 || d->H_q <= 0 || d->W <= 0) return 0;
  return moment_ws(d).total;
}

extern "C" kvm_status kvm_moment_alpha(const kvm_moment_desc* d, const void* Qwin, const void* K, float* alpha,
                                       void* ws, size_t ws_bytes, void* stream) {
  kvm_status st = check_moment_desc(d);
  if (st != KVM_OK) return st;
  KVM_REQUIRE(d->H_q > 0 && d->H_q % d->H_kv == 0, KVM_ERR_SHAPE, "H_q %d not a multiple of H_kv %d", d->H_q, d->H_kv);
  KVM_REQUIRE(d->W >= 1 && d->W <= d->L, KVM_ERR_RANGE, "window %d outside [1, L]", d->W);
  const int G = d->H_q / d->H_kv;
  KVM_REQUIRE(d->W * G <= 4 * kAlphaQPW * 32, KVM_ERR_SHAPE, "W * G = %d exceeds %d", d->W * G, 4 * kAlphaQPW * 32);
  KVM_REQUIRE(d->scale > 0.f, KVM_ERR_RANGE, "scale %g must be positive", d->scale);
  KVM_PTR_ALIGNED(Qwin); KVM_PTR_ALIGNED(K); KVM_PTR_ALIGNED(alpha);
  {
    long long ts, hs, bs;
    strides(d, ts, hs, bs);
    KVM_REQUIRE(((long long)(d->L + 2048) * ts + d->d) * 2 < 0x7fffffffLL, KVM_ERR_RANGE,
                "one (sequence, KV head) of K spans more than 2 GiB (L %d)", d->L);
  }
  const MomentWs w = moment_ws(d);
  KVM_REQUIRE(ws != nullptr && ws_bytes >= w.total, KVM_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  KVM_ALIGNED(ws);
  st = require_gfx950();
  if (st != KVM_OK) return st;
  AlphaArgs a{};
  a.Q = static_cast<const uint16_t*>(Qwin);
  a.K = static_cast<const uint16_t*>(K);
  a.alpha = alpha;
  a.part = reinterpret_cast<float2*>(static_cast<char*>(ws) + w.part);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(ws) + w.lse);
  a.L = d->L; a.H_q = d->H_q; a.H_kv = d->H_kv; a.W = d->W; a.G = G; a.WG = d->W * G;
  const int chunk = alpha_chunk(d->L, d->b * d->H_kv);
  a.n_chunks = (d->L + chunk - 1) / chunk;
  strides(d, a.tok_stride, a.head_stride, a.batch_stride);
  a.scale_log2 = d->scale * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(a.n_chunks, d->b * d->H_kv);
  const dim3 mgrid(d->b * d->H_kv);
  if (d->d == 128 && chunk == 2048) {
    hipLaunchKernelGGL((moment_alpha_kernel<128, 1, 2048>), grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(alpha_merge_kernel, mgrid, dim3(256), 0, s, a);
    hipLaunchKernelGGL((moment_alpha_kernel<128, 2, 2048>), grid, dim3(256), 0, s, a);
  } else if (d->d == 128) {
    hipLaunchKernelGGL((moment_alpha_kernel<128, 1, 512>), grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(alpha_merge_kernel, mgrid, dim3(256), 0, s, a);
    hipLaunchKernelGGL((moment_alpha_kernel<128, 2, 512>), grid, dim3(256), 0, s, a);
  } else if (chunk == 2048) {
    hipLaunchKernelGGL((moment_alpha_kernel<64, 1, 2048>), grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(alpha_merge_kernel, mgrid, dim3(256), 0, s, a);
    hipLaunchKernelGGL((moment_alpha_kernel<64, 2, 2048>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((moment_alpha_kernel<64, 1, 512>), grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(alpha_merge_kernel, mgrid, dim3(256), 0, s, a);
    hipLaunchKernelGGL((moment_alpha_kernel<64, 2, 512>), grid, dim3(256), 0, s, a);
  }
  return check_hip(hipGetLastError(), "moment alpha launch");
}

extern "C" kvm_status kvm_moment_score(const kvm_moment_desc* d, const void* K, const void* V, const float* alpha,
                                       const int32_t* n_e, const float* s_k, const float* s_v, const float* S,
                                       float* score, void* stream) {
  kvm_status st = check_moment_desc(d);
  if (st != KVM_OK) return st;
  KVM_PTR_ALIGNED(K); KVM_PTR_ALIGNED(V); KVM_PTR_ALIGNED(alpha); KVM_PTR_ALIGNED(n_e);
  KVM_PTR_ALIGNED(s_k); KVM_PTR_ALIGNED(s_v); KVM_PTR_ALIGNED(S); KVM_PTR_ALIGNED(score);
  {
    long long ts, hs, bs;
    strides(d, ts, hs, bs);
    KVM_REQUIRE(((long long)(d->L + 2048) * ts + d->d) * 2 < 0x7fffffffLL, KVM_ERR_RANGE,
                "one (sequence, KV head) of K/V spans more than 2 GiB (L %d)", d->L);
  }
  st = require_gfx950();
  if (st != KVM_OK) return st;
  ScoreArgs a{};
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.alpha = alpha; a.n_e = n_e; a.s_k = s_k; a.s_v = s_v; a.S = S; a.score = score;
  a.L = d->L; a.H_kv = d->H_kv;
  strides(d, a.tok_stride, a.head_stride, a.batch_stride);
  a.inv_sqrt_d = 1.f / sqrtf((float)d->d);
  const bool wide = (long long)((d->L + 1023) / 1024) * d->b * d->H_kv >= 256;
  const int keys = wide ? 1024 : 256;
  const dim3 grid((d->L + keys - 1) / keys, d->b * d->H_kv);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->d == 128) {
    if (wide) hipLaunchKernelGGL((moment_score_kernel<128, 1024>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((moment_score_kernel<128, 256>), grid, dim3(256), 0, s, a);
  } else {
    if (wide) hipLaunchKernelGGL((moment_score_kernel<64, 1024>), grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((moment_score_kernel<64, 256>), grid, dim3(128), 0, s, a);
  }
  return check_hip(hipGetLastError(), "moment score launch");
}

extern "C" kvm_status kvm_moment_readout(const kvm_mread_desc* d, const void* q, const float* o_R,
                                         const float* lse_R, const int32_t* n_e, const float* s_k,
                                         const float* s_v, const float* S, float* o, void* stream) {
  KVM_PTR(d);
  KVM_REQUIRE(d->b > 0 && d->H_q > 0 && d->H_kv > 0 && d->H_q % d->H_kv == 0, KVM_ERR_SHAPE,
              "b, H_q, H_kv positive with H_q a multiple of H_kv required");
  KVM_REQUIRE(d->d == 64 || d->d == 128, KVM_ERR_SHAPE, "head dim %d not in {64, 128}", d->d);
  KVM_REQUIRE(d->dtype == KVM_F32 || d->dtype == KVM_BF16, KVM_ERR_DTYPE, "dtype %d", d->dtype);
  KVM_REQUIRE(d->H_q / d->H_kv <= 64, KVM_ERR_SHAPE, "group size %d exceeds 64", d->H_q / d->H_kv);
  KVM_PTR_ALIGNED(q); KVM_PTR_ALIGNED(o_R); KVM_PTR_ALIGNED(lse_R); KVM_PTR_ALIGNED(n_e);
  KVM_PTR_ALIGNED(s_k); KVM_PTR_ALIGNED(s_v); KVM_PTR_ALIGNED(S); KVM_PTR_ALIGNED(o);
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;
  const int G = d->H_q / d->H_kv;
  const size_t smem = (size_t)(G * d->d + G) * sizeof(float);
  const dim3 grid(d->H_kv, d->b);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->dtype == KVM_BF16)
    hipLaunchKernelGGL(moment_readout_kernel<uint16_t>, grid, dim3(256), smem, s, static_cast<const uint16_t*>(q),
                       o_R, lse_R, n_e, s_k, s_v, S, o, d->H_q, d->H_kv, d->d, d->scale);
  else
    hipLaunchKernelGGL(moment_readout_kernel<float>, grid, dim3(256), smem, s, static_cast<const float*>(q), o_R,
                       lse_R, n_e, s_k, s_v, S, o, d->H_q, d->H_kv, d->d, d->scale);
  return check_hip(hipGetLastError(), "moment readout launch");
}
