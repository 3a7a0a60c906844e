// A8 + A9 (+ V3): split-K decode attention over the retained cache, merged with the
// online-softmax identity, plus the latent-memory (or moment) read-out.
//
// Attention states: each block reduces one slot range of one (sequence, KV head) to a
// state (a_c, lse_c) per query head of the GQA group -- the attention output and the log
// of its normaliser [ASM, Method: attention state (a, Z)].  The last block to finish for a
// (sequence, KV head) merges the states in chunk order: lse = log sum exp(lse_c),
// a = sum exp(lse_c - lse) a_c [ASM, Method: online-softmax merge], then adds the read-out
// o = a + g(q) m(q) with m(q) = M phi(q) / (b . phi(q) + eps), g(q) = sigmoid(w_g . q)
// [IM 2.B, output], or mixes with the moment estimate [MKV 2, 4].
//
// Cache layout: Kc [b, H_kv, cap, d] (slot-major), Vc [b, H_kv, d, cap] (dim-major).
//
// bf16, d = 128 (matrix-core path): a wave takes 32-slot tiles.  S = q K^T runs on
// v_mfma_f32_16x16x32_bf16 with the G query heads as rows (padded to 16) and K read
// straight from HBM into B-operand registers (4 lanes x 16 bytes = 64 contiguous bytes of
// a row per instruction).  P V runs on the same instruction with P (bf16 hi + lo, 16-bit
// accurate) as the A operand and the dim-major V cache as the B operand: each lane reads
// 8 consecutive slots of one dim, 16 contiguous bytes.  Loads roll: the next tile's K
// loads are issued into the K registers as soon as S is computed and its V loads as soon
// as P V is done, so one tile of loads is always in flight per wave.  K/V bytes are read
// once for all G heads.  Other shapes (fp32, d = 64) use an FMA path.
//
// Two kernels: the attention kernel writes one partial state per block; the merge kernel
// (one block per 32 output dims of a (sequence, KV head)) merges them in chunk order and
// computes the read-out rows M phi(q) for its dims.  The kernel boundary makes the partial
// states visible across the chip's XCDs; a per-block release/acquire handshake inside one
// kernel costs an L2 write-back and invalidate per block on this part.
#include "common.hpp"

namespace kvm {

struct DecodeArgs {
  const void* q;
  const void* k_new;
  const void* v_new;
  const int32_t* append_slot;
  void* Kc;
  void* Vc;
  const int32_t* len;
  const float* M;
  const float* bvec;
  const void* w_g;
  const int32_t* n_e;
  const float* s_k;
  const float* s_v;
  const float* S;
  const float* rmat;  // read-out matrix: M (memory) or S (moments), chosen on the host
  float* o;
  float* lse;
  float* part_a;    // [b, H_kv, n_split, G, D]
  float* part_lse;  // [b, H_kv, n_split, G]
  float* num;       // [b, H_kv, G, D]   read-out numerator rows
  float* red;       // [b, H_kv, 2, G]   read-out denominator (+eps) and gate, or s_k . q
  int b, H_q, H_kv, cap, n_split, mode;
  float scale, eps;
};

static constexpr float kLog2e = 1.4426950408889634f;
static constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float xor_lane(float x, int mask) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute((__lane_id() ^ mask) << 2, __float_as_int(x)));
}

struct Span {
  int n, app, j0, j1;
};

// tokens attended, append slot and this block's slot range (multiples of `align`)
__device__ __forceinline__ Span block_span(const DecodeArgs& a, int bb, int c, int align) {
  Span s;
  const int len0 = a.len[bb];
  if (!a.k_new) { s.n = len0; s.app = -1; }
  else if (a.append_slot) { s.n = len0; s.app = a.append_slot[bb]; }
  else { s.n = len0 + 1; s.app = len0; }
  s.n = min(max(s.n, 0), a.cap);
  if (s.app < 0 || s.app >= a.cap) s.app = -1;
  int per = (s.n + a.n_split - 1) / a.n_split;
  per = (per + align - 1) / align * align;
  s.j0 = c * per;
  s.j1 = min(s.n, s.j0 + per);
  return s;
}

// ------------------------------------------------------------------ block partial state
// Inputs in LDS: per wave w and head h the running max s_m (log2 units, scaled logits),
// the sum s_l and the unnormalised accumulator s_acc[w][h][:].  Writes (a_c, lse_c).
template <int D, int G, int NW>
__device__ __forceinline__ void write_partial(const DecodeArgs& a, int c, int g, int bb, float (*s_m)[G],
                                              float (*s_l)[G], float (*s_acc)[G][D]) {
  constexpr int NT = NW * 64;
  const size_t pair = (size_t)bb * a.H_kv + g;
  float* pa = a.part_a + (pair * a.n_split + c) * (size_t)(G * D);
  for (int i = threadIdx.x; i < G * D; i += NT) {
    const int h = i / D, dd = i % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_m[w][h]);
    float L = 0.f, A = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = exp2f(s_m[w][h] - mx);
        L = fmaf(s_l[w][h], f, L);
        A = fmaf(s_acc[w][h][dd], f, A);
      }
    }
    pa[i] = L > 0.f ? A / L : 0.f;
    if (dd == 0) a.part_lse[(pair * a.n_split + c) * G + h] = L > 0.f ? (mx + log2f(L)) * kLn2 : -INFINITY;
  }
}

// ------------------------------------------------------------------ read-out inputs
// Run by every attention block before its tile loop: the block's slice of read-out rows
// num[h][r] = Mat[r] . feat_h (feat = phi(q) for the memory, q for the moments), and in
// block 0 the per-head scalars (b . phi(q) + eps and the gate sigmoid(w_g . q), or s_k . q).
// The row loads are issued by the caller before the first K/V tile, so their latency
// overlaps the K/V stream.
template <int D>
struct ReadoutRegs {
  float4 m0, m1;   // 8 consecutive floats of one Mat row
};

template <typename T, int D, int G, int NT>
__device__ __forceinline__ ReadoutRegs<D> readout_load(const DecodeArgs& a, int c, size_t pair) {
  ReadoutRegs<D> r;
  r.m0 = r.m1 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (a.mode == KVM_READ_NONE) return r;
  constexpr int TPR = D / 8;             // threads per row
  const int rps = (D + a.n_split - 1) / a.n_split;
  const int row = c * rps + threadIdx.x / TPR;
  if (threadIdx.x / TPR < rps && row < D && threadIdx.x < NT) {
    const float* p = a.rmat + pair * (size_t)(D * D) + (size_t)row * D + (threadIdx.x % TPR) * 8;
    r.m0 = *reinterpret_cast<const float4*>(p);
    r.m1 = *reinterpret_cast<const float4*>(p + 4);
  }
  return r;
}

// Read-out rows of this block: num[h][row] = M_row . feat(q_h) for its slice of rows,
// feat = phi (memory) or identity (moments); split 0 also writes the per-head scalars
// (b . phi(q) + eps and the gate, or s_k . q).  Every thread derives the features it needs
// from q directly (q is a few KB and cached), so no LDS staging and no block barrier
// hold back the waves whose K/V loads are already in flight.
template <typename T, int D, int G, int NT>
__device__ __forceinline__ void readout_compute(const DecodeArgs& a, int c, int g, size_t pair, const T* qp,
                                                const ReadoutRegs<D>& r) {
  if (a.mode == KVM_READ_NONE) return;
  const bool mem = a.mode == KVM_READ_MEMORY;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int TPR = D / 8;
  static_assert(TPR == 8 || TPR == 16, "row split");
  constexpr int N = Vec16<T>::N;
  const int rps = (D + a.n_split - 1) / a.n_split;
  constexpr int RPP = NT / TPR;          // rows per pass
  const int c0 = (tid % TPR) * 8;
  float f[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e0 = 0; e0 < 8; e0 += N) {
      float x[N];
      Vec16<T>::load(qp + h * D + c0 + e0, x);
#pragma unroll
      for (int e = 0; e < N; ++e) f[h][e0 + e] = mem ? phi_f(x[e]) : x[e];
    }
  for (int pass = 0; pass * RPP < rps; ++pass) {
    const int rl = pass * RPP + tid / TPR, row = c * rps + rl;
    float mv[8] = {r.m0.x, r.m0.y, r.m0.z, r.m0.w, r.m1.x, r.m1.y, r.m1.z, r.m1.w};
    if (pass > 0) {   // rows beyond the first pass (few split blocks): load them now
      float4 m0 = make_float4(0.f, 0.f, 0.f, 0.f), m1 = m0;
      if (rl < rps && row < D) {
        const float* p = a.rmat + pair * (size_t)(D * D) + (size_t)row * D + c0;
        m0 = *reinterpret_cast<const float4*>(p);
        m1 = *reinterpret_cast<const float4*>(p + 4);
      }
      mv[0] = m0.x; mv[1] = m0.y; mv[2] = m0.z; mv[3] = m0.w;
      mv[4] = m1.x; mv[5] = m1.y; mv[6] = m1.z; mv[7] = m1.w;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) x = fmaf(mv[e], f[h][e], x);
      x = group_sum<TPR>(x);
      if (tid % TPR == 0 && rl < rps && row < D) a.num[(pair * G + h) * D + row] = x;
    }
  }
  if (c == 0) {
    for (int h = wave; h < G; h += NT / 64) {
      float x0 = 0.f, x1 = 0.f;
      for (int k = lane; k < D; k += 64) {
        const float qv = load_scalar<T>(qp + h * D + k);
        if (mem) {
          x0 = fmaf(a.bvec[pair * D + k], phi_f(qv), x0);
          const T* wg = reinterpret_cast<const T*>(a.w_g) + (size_t)(g * G + h) * D;
          x1 = fmaf(load_scalar<T>(wg + k), qv, x1);
        } else {
          x0 = fmaf(a.s_k[pair * D + k], qv, x0);
        }
      }
      x0 = wave_sum(x0);
      x1 = wave_sum(x1);
      if (lane == 0) {
        a.red[(pair * 2 + 0) * G + h] = mem ? x0 + a.eps : x0;
        a.red[(pair * 2 + 1) * G + h] = sigmoid_f(x1);
      }
    }
  }
}

// ------------------------------------------------------------------ merge
// grid (D / 32, H_kv, b), 32 * G threads: thread (h, dim) merges the n_split partial states
// of one output element in chunk order and adds the read-out.  One round of loads.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const int rb = blockIdx.x, g = blockIdx.y, bb = blockIdx.z;
  const int h = threadIdx.x >> 5, dd = rb * 32 + (threadIdx.x & 31);
  if (h >= G) return;
  const size_t pair = (size_t)bb * a.H_kv + g;
  const float* pl = a.part_lse + pair * a.n_split * G + h;
  const float* pa = a.part_a + pair * a.n_split * (size_t)(G * D) + (size_t)h * D + dd;
  // every load first: the first 8 partial states and the read-out values, in one round
  float lv[8], av[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lv[e] = e < a.n_split ? pl[e * G] : -INFINITY;
    av[e] = e < a.n_split ? pa[(size_t)e * G * D] : 0.f;
  }
  float num = 0.f, r0 = 1.f, r1 = 0.f, sv = 0.f;
  int ne = 0;
  if (a.mode != KVM_READ_NONE) {
    num = a.num[(pair * G + h) * D + dd];
    r0 = a.red[(pair * 2 + 0) * G + h];
    r1 = a.red[(pair * 2 + 1) * G + h];
    if (a.mode == KVM_READ_MOMENTS) {
      sv = a.s_v[pair * D + dd];
      ne = a.n_e[pair];
    }
  }
  // online merge of the partial states in chunk order, 8 at a time
  float mx = -INFINITY, z = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < a.n_split; c0 += 8) {
    if (c0 > 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int cc = c0 + e;
        lv[e] = cc < a.n_split ? pl[cc * G] : -INFINITY;
        av[e] = cc < a.n_split ? pa[(size_t)cc * G * D] : 0.f;
      }
    }
    float gm = lv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) gm = fmaxf(gm, lv[e]);
    const float nm = fmaxf(mx, gm);
    if (nm != -INFINITY) {
      const float f = mx == -INFINITY ? 0.f : __expf(mx - nm);
      z *= f;
      acc *= f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float w = lv[e] == -INFINITY ? 0.f : __expf(lv[e] - nm);
        z += w;
        acc = fmaf(w, av[e], acc);
      }
      mx = nm;
    }
  }
  float lse = -INFINITY, o = 0.f;
  if (mx != -INFINITY && z > 0.f) {
    lse = mx + __logf(z);
    o = acc / z;
  }
  if (a.mode == KVM_READ_MEMORY) {
    o = fmaf(r1, num / r0, o);
  } else if (a.mode == KVM_READ_MOMENTS && ne > 0) {
    const float inv = 1.f / (float)ne;
    const float fE = sv * inv + a.scale * (num - sv * r0 * inv) * inv;
    const float logZ = __logf((float)ne) + a.scale * r0 * inv;
    const float w = sigmoid_f(lse - logZ);
    o = w * o + (1.f - w) * fE;
  }
  a.o[((size_t)bb * a.H_q + g * G + h) * D + dd] = o;
  if (a.lse && dd == 0) a.lse[(size_t)bb * a.H_q + g * G + h] = lse;
}

// ------------------------------------------------------------------ FMA path (any dtype, D)
template <typename T, int D, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_fma_kernel(DecodeArgs a) {
  constexpr int EPL = Vec16<T>::N;   // elements per lane (16 bytes)
  constexpr int LPT = D / EPL;       // lanes per token row
  constexpr int TPI = 64 / LPT;      // token rows per wave instruction
  const int c = blockIdx.x, g = blockIdx.y, bb = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPT, grp = lane / LPT;

  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_acc[NW][G][D];

  const Span sp = block_span(a, bb, c, 1);
  const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)bb * a.H_q + (size_t)g * G) * D;
  const size_t cache_off = ((size_t)bb * a.H_kv + g) * (size_t)a.cap * D;
  T* Kp = reinterpret_cast<T*>(a.Kc) + cache_off;
  T* Vt = reinterpret_cast<T*>(a.Vc) + cache_off;   // [D][cap]
  const T* kn = a.k_new ? reinterpret_cast<const T*>(a.k_new) + ((size_t)bb * a.H_kv + g) * D : nullptr;
  const T* vn = a.v_new ? reinterpret_cast<const T*>(a.v_new) + ((size_t)bb * a.H_kv + g) * D : nullptr;
  {
    const size_t pair = (size_t)bb * a.H_kv + g;
    const ReadoutRegs<D> rr = readout_load<T, D, G, NW * 64>(a, c, pair);
    readout_compute<T, D, G, NW * 64>(a, c, g, pair, qp, rr);
  }

  float qf[G][EPL];
  const float qs = a.scale * kLog2e;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float t[EPL];
    Vec16<T>::load(qp + h * D + sub * EPL, t);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[h][e] = t[e] * qs;
  }
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  for (int j = sp.j0 + wave * TPI + grp; j < sp.j1; j += NW * TPI) {
    const bool is_new = (j == sp.app);
    float kf[EPL], vf[EPL];
    if (is_new) {
      const uint4 kraw = *reinterpret_cast<const uint4*>(kn + sub * EPL);
      *reinterpret_cast<uint4*>(Kp + (size_t)j * D + sub * EPL) = kraw;
      Vec16<T>::unpack(kraw, kf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const T v = vn[sub * EPL + e];
        Vt[(size_t)(sub * EPL + e) * a.cap + j] = v;
        vf[e] = load_scalar<T>(&v);
      }
    } else {
      Vec16<T>::load(Kp + (size_t)j * D + sub * EPL, kf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) vf[e] = load_scalar<T>(Vt + (size_t)(sub * EPL + e) * a.cap + j);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s = fmaf(qf[h][e], kf[e], s);
      s = group_sum<LPT>(s);
      const float mn = fmaxf(m[h], s);
      const float cf = exp2f(m[h] - mn);
      const float p = exp2f(s - mn);
      l[h] = fmaf(l[h], cf, p);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(acc[h][e], cf, p * vf[e]);
      m[h] = mn;
    }
  }
  // merge the TPI lane groups of the wave
#pragma unroll
  for (int msk = LPT; msk < 64; msk <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m2 = xor_lane(m[h], msk);
      const float l2 = xor_lane(l[h], msk);
      const float mn = fmaxf(m[h], m2);
      const float f1 = mn == -INFINITY ? 0.f : exp2f(m[h] - mn);
      const float f2 = mn == -INFINITY ? 0.f : exp2f(m2 - mn);
      l[h] = l[h] * f1 + l2 * f2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float a2 = xor_lane(acc[h][e], msk);
        acc[h][e] = acc[h][e] * f1 + a2 * f2;
      }
      m[h] = mn;
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][h][sub * EPL + e] = acc[h][e];
      if (sub == 0) { s_m[wave][h] = m[h]; s_l[wave][h] = l[h]; }
    }
  }
  __syncthreads();
  write_partial<D, G, NW>(a, c, g, bb, s_m, s_l, s_acc);
}

// ------------------------------------------------------------------ matrix-core tile helpers
struct TileRegs {
  uint4 k[2][4];   // K rows of slots t0 + gq*16 + m16, dims cc*32 + kg*8 .. +8
  uint4 v[8];      // V dims dt*16 + m16, slots t0 + kg*8 .. +8
};

__device__ __forceinline__ void tile_load_k(TileRegs& T, int t0, const Span& sp, const uint16_t* Kp,
                                            const uint16_t* kn, int m16, int kg) {
  constexpr int D = 128;
#pragma unroll
  for (int gq = 0; gq < 2; ++gq) {
    const int t = t0 + gq * 16 + m16;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < sp.j1) {
        const uint16_t* src = (t == sp.app) ? kn + cc * 32 + kg * 8 : Kp + (size_t)t * D + cc * 32 + kg * 8;
        v = *reinterpret_cast<const uint4*>(src);
      }
      T.k[gq][cc] = v;
    }
  }
}

__device__ __forceinline__ void tile_load_v(TileRegs& T, int t0, const Span& sp, const uint16_t* Vt, int cap,
                                            int m16, int kg) {
  const int tv = t0 + kg * 8;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (tv < sp.j1) v = *reinterpret_cast<const uint4*>(Vt + (size_t)(dt * 16 + m16) * cap + tv);
    T.v[dt] = v;
  }
}

// S = q K^T for slots t0 + gq*16 + m16
__device__ __forceinline__ void tile_scores(const TileRegs& T, const bf16x8_t (&qa)[4], f32x4_t (&sc)[2]) {
#pragma unroll
  for (int gq = 0; gq < 2; ++gq) {
    sc[gq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      bf16x8_t kb;
      __builtin_memcpy(&kb, &T.k[gq][cc], 16);
      sc[gq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[cc], kb, sc[gq], 0, 0, 0);
    }
  }
}

// online softmax of one tile's scores, then acc = acc * cf + P V
template <int G>
__device__ __forceinline__ void tile_pv(const TileRegs& T, const f32x4_t (&sc)[2], int t0, const Span& sp,
                                        const uint16_t* vn, float qs, int m16, int kg, bool real_rows,
                                        uint32_t (*s_p)[8][16], float (&m)[4], float (&l)[4], f32x4_t (&acc)[8]) {
  // online softmax on the real head rows (4*kg + i < G)
  float cf[4];
  const bool ok0 = t0 + m16 < sp.j1, ok1 = t0 + 16 + m16 < sp.j1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = ok0 ? sc[0][i] * qs : -INFINITY;
    const float x1 = ok1 ? sc[1][i] * qs : -INFINITY;
    const float mx = group_max<16>(fmaxf(x0, x1));
    const float mn = fmaxf(m[i], mx);
    const float msafe = mn == -INFINITY ? 0.f : mn;
    cf[i] = exp2f(m[i] - msafe);
    const float p0 = exp2f(x0 - msafe), p1 = exp2f(x1 - msafe);
    l[i] = fmaf(l[i], cf[i], p0 + p1);
    m[i] = mn;
    // P (bf16 hi + lo) -> LDS as [row][slot]
    if (real_rows && 4 * kg + i < G) {
      const uint32_t h0 = f32_to_bf16_bits(p0), h1 = f32_to_bf16_bits(p1);
      const uint32_t lo0 = f32_to_bf16_bits(p0 - __uint_as_float(h0 << 16));
      const uint32_t lo1 = f32_to_bf16_bits(p1 - __uint_as_float(h1 << 16));
      uint16_t* ph = reinterpret_cast<uint16_t*>(&s_p[0][4 * kg + i][0]);
      uint16_t* pl = reinterpret_cast<uint16_t*>(&s_p[1][4 * kg + i][0]);
      ph[m16] = (uint16_t)h0; ph[16 + m16] = (uint16_t)h1;
      pl[m16] = (uint16_t)lo0; pl[16 + m16] = (uint16_t)lo1;
    }
  }
  // A operand of P V: lane (row m16, kg) holds P[m16][kg*8 .. +8]
  uint4 phv = make_uint4(0, 0, 0, 0), plv = make_uint4(0, 0, 0, 0);
  if (m16 < G) {
    phv = *reinterpret_cast<const uint4*>(&s_p[0][m16][kg * 4]);
    plv = *reinterpret_cast<const uint4*>(&s_p[1][m16][kg * 4]);
  }
  bf16x8_t pha, pla;
  __builtin_memcpy(&pha, &phv, 16);
  __builtin_memcpy(&pla, &plv, 16);
  // V fragment fix-ups: zero slots >= j1, insert the appended token
  const int tv = t0 + kg * 8;
  const int valid = sp.j1 - tv;
  const int ap = sp.app - tv;
  const bool fix = valid < 8 || (ap >= 0 && ap < 8);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    uint4 v = T.v[dt];
    if (fix) {
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t val = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu);
        if (e == ap) val = vn[dt * 16 + m16];
        if (e >= valid) val = 0;
        w[e >> 1] = (e & 1) ? ((w[e >> 1] & 0xffffu) | (val << 16)) : ((w[e >> 1] & 0xffff0000u) | val);
      }
      v = make_uint4(w[0], w[1], w[2], w[3]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[dt][i] *= cf[i];
    bf16x8_t vb;
    __builtin_memcpy(&vb, &v, 16);
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pha, vb, acc[dt], 0, 0, 0);
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pla, vb, acc[dt], 0, 0, 0);
  }
}

// ------------------------------------------------------------------ matrix-core path
// bf16, D = 128.  One 32-slot tile per wave iteration.
#ifndef KVM_DECODE_WPE
#define KVM_DECODE_WPE 2
#endif
constexpr int WPE = KVM_DECODE_WPE;
template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int D = 128, NW = 4, TILE = 32;
  static_assert(G <= 8, "G");
  const int c = blockIdx.x, g = blockIdx.y, bb = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, kg = lane >> 4;

  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_acc[NW][G][D];
  __shared__ uint32_t s_p[NW][2][8][TILE / 2];   // per wave: hi/lo, head row, slot pairs

  const size_t pair = (size_t)bb * a.H_kv + g;
  const ReadoutRegs<D> rregs = readout_load<uint16_t, D, G, NW * 64>(a, c, pair);
  // split boundaries on 64-slot multiples: with a cap of a multiple of 64 every 128-byte
  // line of a V row belongs to one block
  const Span sp = block_span(a, bb, c, 2 * TILE);
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)bb * a.H_q + (size_t)g * G) * D;
  uint16_t* Kp = reinterpret_cast<uint16_t*>(a.Kc) + pair * (size_t)a.cap * D;
  uint16_t* Vt = reinterpret_cast<uint16_t*>(a.Vc) + pair * (size_t)a.cap * D;
  const uint16_t* kn = a.k_new ? reinterpret_cast<const uint16_t*>(a.k_new) + pair * D : nullptr;
  const uint16_t* vn = a.v_new ? reinterpret_cast<const uint16_t*>(a.v_new) + pair * D : nullptr;

  // A operand of S = q K^T: lane (row m16, k group kg) holds q[m16][cc*32 + kg*8 .. +8]
  bf16x8_t qa[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m16 < G) v = *reinterpret_cast<const uint4*>(qp + m16 * D + cc * 32 + kg * 8);
    __builtin_memcpy(&qa[cc], &v, 16);
  }
  const float qs = a.scale * kLog2e;
  float m[4], l[4];
  f32x4_t acc[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m[i] = -INFINITY; l[i] = 0.f; }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool real_rows = 4 * kg < G;

  // the block that owns the appended slot writes it into the caches
  if (sp.app >= sp.j0 && sp.app < sp.j1 && wave == 0) {
    for (int i = lane; i < D; i += 64) {
      Kp[(size_t)sp.app * D + i] = kn[i];
      Vt[(size_t)i * a.cap + sp.app] = vn[i];
    }
  }

  // Rolling loads: the next tile's K goes into the K registers once S is computed, its V
  // into the V registers once P V is done, so a tile of loads stays in flight per wave.
  TileRegs ta;
  int t0 = sp.j0 + wave * TILE;
  if (t0 < sp.j1) {
    tile_load_k(ta, t0, sp, Kp, kn, m16, kg);
    tile_load_v(ta, t0, sp, Vt, a.cap, m16, kg);
  }
  readout_compute<uint16_t, D, G, NW * 64>(a, c, g, pair, qp, rregs);
  for (; t0 < sp.j1; t0 += NW * TILE) {
    const int tn = t0 + NW * TILE;
    f32x4_t sc[2];
    tile_scores(ta, qa, sc);
    if (tn < sp.j1) tile_load_k(ta, tn, sp, Kp, kn, m16, kg);
    tile_pv<G>(ta, sc, t0, sp, vn, qs, m16, kg, real_rows, s_p[wave], m, l, acc);
    if (tn < sp.j1) tile_load_v(ta, tn, sp, Vt, a.cap, m16, kg);
  }
  // wave state -> LDS: rows 4*kg + i < G live in lanes of group kg
#pragma unroll
  for (int i = 0; i < 4; ++i) l[i] = group_sum<16>(l[i]);
  if (real_rows) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * kg + i;
      if (h < G) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) s_acc[wave][h][dt * 16 + m16] = acc[dt][i];
        if (m16 == 0) { s_m[wave][h] = m[i]; s_l[wave][h] = l[i]; }
      }
    }
  }
  __syncthreads();
  write_partial<D, G, NW>(a, c, g, bb, s_m, s_l, s_acc);
}

__global__ void len_add_kernel(int32_t* len, int b, int delta) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < b) len[i] += delta;
}

static int auto_split(const kvm_decode_desc* d) {
  if (d->n_split > 0) return d->n_split;
  const int pairs = d->b * d->H_kv;
  int s = (512 + pairs - 1) / pairs;
  s = std::min(s, std::max(1, d->cap / 128));
  return std::max(1, std::min(s, 64));
}

struct DecodeWs {
  size_t a, lse, num, red, total;
};
static DecodeWs decode_ws(const kvm_decode_desc* d, int ns) {
  const int G = d->H_q / d->H_kv;
  const size_t pairs = (size_t)d->b * d->H_kv;
  DecodeWs w;
  w.a = 0;
  w.lse = align_up(w.a + pairs * ns * G * d->d * sizeof(float), 256);
  w.num = align_up(w.lse + pairs * ns * G * sizeof(float), 256);
  w.red = align_up(w.num + pairs * G * d->d * sizeof(float), 256);
  w.total = align_up(w.red + pairs * 2 * G * sizeof(float), 256);
  return w;
}

template <typename T, int D, int G>
static void launch_decode(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.n_split, a.H_kv, a.b);
  if constexpr (std::is_same<T, uint16_t>::value && D == 128)
    hipLaunchKernelGGL((decode_mfma_kernel<G>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((decode_fma_kernel<T, D, G, 4>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL((decode_merge_kernel<D, G>), dim3(D / 32, a.H_kv, a.b), dim3(32 * G), 0, st, a);
}

template <typename T, int D>
static bool dispatch_g(int G, const DecodeArgs& a, hipStream_t st) {
  switch (G) {
    case 1: launch_decode<T, D, 1>(a, st); return true;
    case 2: launch_decode<T, D, 2>(a, st); return true;
    case 4: launch_decode<T, D, 4>(a, st); return true;
    case 8: launch_decode<T, D, 8>(a, st); return true;
  }
  return false;
}

}  // namespace kvm

using namespace kvm;

extern "C" size_t kvm_decode_workspace_size(const kvm_decode_desc* d) {
  if (!d || d->b <= 0 || d->H_kv <= 0 || d->H_q <= 0 || d->d <= 0 || d->cap <= 0) return 0;
  return decode_ws(d, auto_split(d)).total;
}

extern "C" kvm_status kvm_decode_attn_mem(const kvm_decode_desc* d, const void* q, const void* k_new,
                                          const void* v_new, const int32_t* append_slot, void* Kc,
                                          void* Vc, const int32_t* len, const float* M,
                                          const float* bvec, const void* w_g, const int32_t* n_e,
                                          const float* s_k, const float* s_v, const float* S,
                                          float* o, float* lse, void* ws, size_t ws_bytes,
                                          void* stream) {
  KVM_PTR(d);
  KVM_REQUIRE(d->b > 0 && d->H_q > 0 && d->H_kv > 0 && d->cap > 0, KVM_ERR_SHAPE,
              "b, H_q, H_kv and cap must be positive");
  KVM_REQUIRE(d->cap % 8 == 0, KVM_ERR_SHAPE, "cap %d is not a multiple of 8", d->cap);
  KVM_REQUIRE(d->d == 64 || d->d == 128, KVM_ERR_SHAPE, "head dim %d not in {64, 128}", d->d);
  KVM_REQUIRE(d->H_q % d->H_kv == 0, KVM_ERR_SHAPE, "H_q %% H_kv != 0");
  const int G = d->H_q / d->H_kv;
  KVM_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, KVM_ERR_SHAPE, "group size %d not in {1,2,4,8}", G);
  KVM_REQUIRE(d->dtype == KVM_F32 || d->dtype == KVM_BF16, KVM_ERR_DTYPE, "dtype %d", d->dtype);
  KVM_REQUIRE(d->mode >= KVM_READ_NONE && d->mode <= KVM_READ_MOMENTS, KVM_ERR_RANGE, "mode %d", d->mode);
  KVM_REQUIRE(d->n_split >= 0 && d->n_split <= 64, KVM_ERR_RANGE, "n_split %d outside [0, 64]", d->n_split);
  KVM_PTR_ALIGNED(q); KVM_PTR_ALIGNED(Kc); KVM_PTR_ALIGNED(Vc); KVM_PTR_ALIGNED(len); KVM_PTR_ALIGNED(o);
  KVM_REQUIRE((k_new == nullptr) == (v_new == nullptr), KVM_ERR_NULL, "k_new and v_new must both be given or both NULL");
  KVM_REQUIRE(append_slot == nullptr || k_new != nullptr, KVM_ERR_NULL, "append_slot needs k_new");
  KVM_OPT_ALIGNED(k_new); KVM_OPT_ALIGNED(v_new); KVM_OPT_ALIGNED(lse);
  if (d->mode == KVM_READ_MEMORY) { KVM_PTR_ALIGNED(M); KVM_PTR_ALIGNED(bvec); KVM_PTR_ALIGNED(w_g); }
  if (d->mode == KVM_READ_MOMENTS) {
    KVM_PTR_ALIGNED(n_e); KVM_PTR_ALIGNED(s_k); KVM_PTR_ALIGNED(s_v); KVM_PTR_ALIGNED(S);
  }
  const int ns = auto_split(d);
  const DecodeWs w = decode_ws(d, ns);
  KVM_REQUIRE(ws != nullptr && ws_bytes >= w.total, KVM_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  KVM_ALIGNED(ws);
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;

  DecodeArgs a{};
  a.q = q; a.k_new = k_new; a.v_new = v_new; a.append_slot = append_slot;
  a.Kc = Kc; a.Vc = Vc; a.len = len; a.M = M; a.bvec = bvec; a.w_g = w_g;
  a.n_e = n_e; a.s_k = s_k; a.s_v = s_v; a.S = S; a.o = o; a.lse = lse;
  a.rmat = d->mode == KVM_READ_MEMORY ? M : S;
  char* base = static_cast<char*>(ws);
  a.part_a = reinterpret_cast<float*>(base + w.a);
  a.part_lse = reinterpret_cast<float*>(base + w.lse);
  a.num = reinterpret_cast<float*>(base + w.num);
  a.red = reinterpret_cast<float*>(base + w.red);
  a.b = d->b; a.H_q = d->H_q; a.H_kv = d->H_kv; a.cap = d->cap; a.n_split = ns; a.mode = d->mode;
  a.scale = d->scale; a.eps = d->eps;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool ok;
  if (d->dtype == KVM_BF16)
    ok = d->d == 128 ? dispatch_g<uint16_t, 128>(G, a, s) : dispatch_g<uint16_t, 64>(G, a, s);
  else
    ok = d->d == 128 ? dispatch_g<float, 128>(G, a, s) : dispatch_g<float, 64>(G, a, s);
  if (!ok) return set_error(KVM_ERR_SHAPE, "unsupported group size");
  return check_hip(hipGetLastError(), "decode kernel launch");
}

extern "C" kvm_status kvm_len_add(int32_t* len, int32_t b, int32_t delta, void* stream) {
  KVM_PTR_ALIGNED(len);
  KVM_REQUIRE(b > 0, KVM_ERR_SHAPE, "b must be positive");
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;
  hipLaunchKernelGGL(len_add_kernel, dim3((b + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), len, b, delta);
  return check_hip(hipGetLastError(), "len_add launch");
}
