// MomentKV eviction during decode: one token per (sequence, KV head) and step leaves a
// fixed pool of P slots, chosen by the moment-informed score and folded into the moments
// [MKV part 1: the sums are updated at every eviction; MKV part 3: score_j = alpha_j ||r_j||].
//
// Per step, for the new token at position p:
//   alpha_j = (1/G) sum over the group's query heads of the new query's softmax weight of
//             pooled token j; the softmax runs over the pool and the new token;
//   r_j     = v_j - s_v/n_e - (S k_j - s_v (s_k . k_j)/n_e) / (n_e sqrt d)  (v_j while n_e = 0);
//   e       = argmin alpha_j ||r_j|| over the slots at positions <= p - R (ties evict the
//             higher position); n_e, s_k, s_v, S take k_e, v_e; the new token takes slot e.
// The new query then attends over the pool with the NC mix (kvm_decode_attn_mem in
// moments mode).
//
// Two kernels:
//   mstream_score_kernel   per (64- or 128-slot chunk, KV head, sequence): the residual norms on
//                          the matrix cores (S' = S~/(n_e sqrt d) as three bf16 terms
//                          against the exact bf16 keys) and the group's logits q_h . k_j
//                          (one more product, queries as rows); advances next_pos
//   mstream_commit_kernel  per (KV head, sequence): log-sum-exp of each head over the
//                          pool and the new token, alpha, the argmin, the rank-1 moment
//                          fold and the new token's K/V written into the freed slot
#include "common.hpp"

namespace kvm {

struct MsArgs {
  const uint16_t* q;      // [b, H_q, D]
  const uint16_t* k_new;  // [b, H_kv, D]
  const uint16_t* v_new;  // [b, H_kv, D]
  uint16_t* Kc;           // [b, H_kv, cap, D] slot-major
  uint16_t* Vc;           // [b, H_kv, D, cap] dim-major
  int32_t* slot_pos;      // [b, H_kv, P]
  int32_t* next_pos;      // [b]
  int32_t* n_e;           // [b, H_kv]
  float* s_k;             // [b, H_kv, D]
  float* s_v;             // [b, H_kv, D]
  float* S;               // [b, H_kv, D, D]
  int32_t* evict_slot;    // [b, H_kv]
  float* lg;              // ws [b, H_kv, G, P]: scale q_h . k_j
  float* rn;              // ws [b, H_kv, P]: ||r_j||
  int H_q, H_kv, G, P, cap, R;
  float scale;            // 1 / sqrt(D)
};

// grid (ceil(P / KEYS), H_kv, b), D / 32 waves; KEYS pool slots per block (64, or 128 where
// that still gives every CU a block: each block splits its KV head's S once, so larger blocks
// repeat that less; 1024-slot pools at batch 4: 36.3 -> 31.7 us per step).  Wave w owns residual dims 32w .. 32w+31
// of 32 slots per tile: C[i][slot] = sum_c S'[i][c] k[slot][c], r = v - v_bar - C, and
// ||r||^2 sums the lane's rows, the two half-waves and the waves.  Wave 0 also forms
// C[h][slot] = q_h . k[slot] with the group's queries as the rows of a fourth product.
template <int D, int KEYS>
__global__ __launch_bounds__(D * 2) void mstream_score_kernel(MsArgs a) {
  constexpr int kMsKeys = KEYS;
  constexpr int KS = D / 16;
  constexpr int NW = D / 32;
  constexpr int NT = kMsKeys / 32;
  constexpr int P = D / 8;              // 16-byte pieces per key row
  constexpr int NLD = kMsKeys / 16;     // 1 KB loads per wave for each of K and V
  static_assert(NLD * NW * 1024 == kMsKeys * D * 2, "the waves' loads cover the block");
  const int c = blockIdx.x, g = blockIdx.y, bb = blockIdx.z;
  const size_t pair = (size_t)bb * a.H_kv + g;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  // the block's K rows [KEYS][P pieces] (swizzled by piece_swz) and V columns [D][KEYS]
  // (dim-major, as in the cache); after the products the K region holds the per-wave sums
  __shared__ __attribute__((aligned(16))) uint32_t s_kb[kMsKeys * D / 2];
  __shared__ __attribute__((aligned(16))) uint32_t s_vb[kMsKeys * D / 2];
  // the step's position advances once per sequence, here; the commit reads next_pos - 1
  if (c == 0 && g == 0 && tid == 0) a.next_pos[bb] += 1;

  const int ne = a.n_e[pair];
  const float inv_n = (ne > 0 ? 1.f : 0.f) / (float)max(ne, 1);   // no branch on the count
  const float* sk = a.s_k + pair * D;
  const float* sv = a.s_v + pair * D;
  // K and V come into LDS by direct buffer-to-LDS loads, 1 KB each, issued right after the
  // S rows so that they travel while S is split.  K slots past the pool read zeros; V
  // slots past it read whatever the rows hold (cap is a multiple of 8, so every row's
  // slots start on a 16-byte boundary) and only reach results that are never written.
  const int k0 = c * kMsKeys;
  const auto rK = make_rsrc(a.Kc + pair * a.cap * D, a.P * D * 2);
  const auto rV = make_rsrc(a.Vc + pair * D * a.cap, D * a.cap * 2);
  // A operands: row i = 32 wave + col of S' (zero while nothing is evicted).  Every load is
  // unconditional; the count only selects the result, so no load waits behind a branch.
  const int i_row = wave * 32 + col;
  bf16x8_t sh[KS], sm[KS], sl3[KS];
  {
    const float* Sr = a.S + (pair * D + i_row) * D;
    const float svi = sv[i_row];
    const float f = inv_n * a.scale;
    float4 s4[KS][2], k4[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        s4[ks][u] = *reinterpret_cast<const float4*>(Sr + ks * 16 + half * 8 + 4 * u);
        k4[ks][u] = *reinterpret_cast<const float4*>(sk + ks * 16 + half * 8 + 4 * u);
      }
    }
    // the block's K and V, issued behind the S rows (the offsets are computed apart from the
    // load builtin's arguments: with a device call inside them the host pass drops the
    // kernel's launch stubs)
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int i = NLD * wave + j;
      const int sl = i * 64 + lane, r = sl / P, q = sl % P;
      const int koff = ((k0 + r) * D + 8 * (q ^ piece_swz<P>(r))) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (__attribute__((address_space(3))) void*)(&s_kb[i * 256]), 16, koff,
                                               0, 0, 0);
      const int bv = i * 1024 + lane * 16;   // byte of the V block
      const int dim = bv / (kMsKeys * 2), sb = bv % (kMsKeys * 2);
      const int voff = (dim * a.cap + k0) * 2 + sb;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (__attribute__((address_space(3))) void*)(&s_vb[i * 256]), 16, voff,
                                               0, 0, 0);
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
      split3_bf16x8(x, sh[ks], sm[ks], sl3[ks]);
    }
  }
  // the group's queries as rows (rows >= G read zeros)
  bf16x8_t qa[KS];
  {
    const auto rq = make_rsrc(a.q + ((size_t)bb * a.H_q + (size_t)g * a.G) * D, a.G * D * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rq, (col * D + ks * 16 + half * 8) * 2, 0, 0);
      __builtin_memcpy(&qa[ks], &v, 16);
    }
  }
  // v_bar of the 16 dims this lane holds in the C layout
  float vbar[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) vbar[j] = sv[wave * 32 + 8 * (j / 4) + 4 * half + (j % 4)] * inv_n;

  // every wave's loads have landed: the block's K and V are in LDS
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const uint16_t* svh = reinterpret_cast<const uint16_t*>(s_vb);
  float ssr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int slot = k0 + t * 32 + col;
    const bool ok = slot < a.P;
    f32x16_t acc, accq;
#pragma unroll
    for (int j = 0; j < 16; ++j) { acc[j] = 0.f; accq[j] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // B operand: slot t*32 + col, dims ks*16 + half*8 .. +8
      const uint4 kv = *reinterpret_cast<const uint4*>(&s_kb[((t * 32 + col) * P + ((2 * ks + half) ^ piece_swz<P>(col))) * 4]);
      bf16x8_t B;
      __builtin_memcpy(&B, &kv, 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sh[ks], B, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sm[ks], B, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sl3[ks], B, acc, 0, 0, 0);
      if (wave == 0) accq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks], B, accq, 0, 0, 0);
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int dim = wave * 32 + 8 * (j / 4) + 4 * half + (j % 4);
      const float r = bf16_to_f32(svh[dim * kMsKeys + t * 32 + col]) - vbar[j] - acc[j];
      ss = fmaf(r, r, ss);
    }
    ssr[t] = ss + shfl_xor32(ss);
    if (wave == 0 && ok) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int h = 8 * (j / 4) + 4 * half + (j % 4);
        if (h < a.G) a.lg[(pair * a.G + h) * a.P + slot] = accq[j] * a.scale;
      }
    }
  }
  __syncthreads();   // every wave is done with the K rows: their LDS takes the sums
  float* s_ss = reinterpret_cast<float*>(s_kb);   // [NW][KEYS]
#pragma unroll
  for (int t = 0; t < NT; ++t) s_ss[wave * kMsKeys + t * 32 + col] = ssr[t];   // both halves: same sum
  __syncthreads();
  for (int i = tid; i < kMsKeys; i += NW * 64) {
    const int j = k0 + i;
    if (j < a.P) {
      float ss = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) ss += s_ss[w * kMsKeys + i];
      a.rn[pair * a.P + j] = sqrtf(ss);
    }
  }
}

// grid (H_kv, b), 256 threads: the eviction of one (sequence, KV head) and its fold.  The
// pool is read in passes of 1024 slots (4 per thread), each pass's loads issued together.
template <int D, int G>
__global__ __launch_bounds__(256) void mstream_commit_kernel(MsArgs a) {
  constexpr int NS = D * D / 1024;   // float4 of S per thread
  constexpr int NPT = 4;             // pool slots per thread and pass
  constexpr int PASS = 256 * NPT;
  const int g = blockIdx.x, bb = blockIdx.y;
  const size_t pair = (size_t)bb * a.H_kv + g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = a.P;
  __shared__ float s_new[G], s_lse[G];
  __shared__ float s_wm[4][G], s_wz[4][G];
  __shared__ float s_ke[D], s_ve[D];
  __shared__ unsigned long long s_best[4];
  __shared__ int s_bslot[4];

  // this pair's S, independent of the choice: loads issued first
  float4* S4 = reinterpret_cast<float4*>(a.S + pair * D * D);
  float4 sr[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) sr[i] = S4[i * 256 + tid];
  const int p = a.next_pos[bb] - 1;
  const float* lgp = a.lg + pair * G * P;

  // the new token's logit per head (one wave per head)
  for (int h = wave; h < G; h += 4) {
    const uint16_t* qh = a.q + ((size_t)bb * a.H_q + (size_t)g * G + h) * D;
    const uint16_t* kn = a.k_new + pair * D;
    float dot = 0.f;
#pragma unroll
    for (int c = lane; c < D; c += 64) dot = fmaf(bf16_to_f32(qh[c]), bf16_to_f32(kn[c]), dot);
    dot = wave_sum(dot);
    if (lane == 0) s_new[h] = dot * a.scale;
  }

  // per head: online (max, sum of exp) over this thread's slots, then over the block
  float m[G], z[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; z[h] = 0.f; }
  for (int j0 = 0; j0 < P; j0 += PASS) {
    float v[G][NPT];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int u = 0; u < NPT; ++u) v[h][u] = lgp[h * P + min(j0 + u * 256 + tid, P - 1)];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = m[h];
#pragma unroll
      for (int u = 0; u < NPT; ++u) mx = j0 + u * 256 + tid < P ? fmaxf(mx, v[h][u]) : mx;
      float zz = mx == -INFINITY ? 0.f : z[h] * __expf(m[h] - mx);
#pragma unroll
      for (int u = 0; u < NPT; ++u) zz += j0 + u * 256 + tid < P ? __expf(v[h][u] - mx) : 0.f;
      m[h] = mx;
      z[h] = zz;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float wm = group_max<64>(m[h]);
    const float wz = wave_sum(wm == -INFINITY ? 0.f : z[h] * __expf(m[h] - wm));
    if (lane == 0) { s_wm[wave][h] = wm; s_wz[wave][h] = wz; }
  }
  __syncthreads();
  if (tid < G) {
    const int h = tid;
    float mx = s_new[h];
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, s_wm[w][h]);
    float zz = __expf(s_new[h] - mx);
    for (int w = 0; w < 4; ++w) zz += s_wm[w][h] == -INFINITY ? 0.f : s_wz[w][h] * __expf(s_wm[w][h] - mx);
    s_lse[h] = mx + __logf(zz);
  }
  __syncthreads();
  float lse[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lse[h] = s_lse[h];

  // alpha, the score and the lowest candidate (ties: the higher position goes)
  const float invG = 1.f / (float)G;
  unsigned long long key = ~0ull;
  int slot = -1;
  for (int j0 = 0; j0 < P; j0 += PASS) {
    float v[G][NPT], r[NPT];
    int ps[NPT];
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int j = min(j0 + u * 256 + tid, P - 1);
#pragma unroll
      for (int h = 0; h < G; ++h) v[h][u] = lgp[h * P + j];
      r[u] = a.rn[pair * P + j];
      ps[u] = a.slot_pos[pair * P + j];
    }
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int j = j0 + u * 256 + tid;
      float al = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) al += __expf(v[h][u] - lse[h]);
      const float sc = al * invG * r[u];
      if (j < P && ps[u] <= p - a.R) {
        const unsigned long long k = ((unsigned long long)order_key(sc) << 32) | (uint32_t)(0x7fffffff - ps[u]);
        if (k < key) { key = k; slot = j; }
      }
    }
  }
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long ok = __shfl_xor(key, off);
    const int os = __shfl_xor(slot, off);
    if (ok < key) { key = ok; slot = os; }
  }
  if (lane == 0) { s_best[wave] = key; s_bslot[wave] = slot; }
  __syncthreads();
  unsigned long long bk = s_best[0];
  int e = s_bslot[0];
  for (int w = 1; w < 4; ++w)
    if (s_best[w] < bk) { bk = s_best[w]; e = s_bslot[w]; }
  if (bk == ~0ull) e = -1;
  if (tid == 0) a.evict_slot[pair] = e;
  if (e < 0) return;   // no candidate: nothing is evicted and the new token is not stored

  // the evicted row, read before the new token overwrites its slot
  uint16_t* kr = a.Kc + (pair * a.cap + e) * D;
  uint16_t* vc = a.Vc + pair * D * a.cap + e;
  if (tid < D) {
    s_ke[tid] = bf16_to_f32(kr[tid]);
    s_ve[tid] = bf16_to_f32(vc[(size_t)tid * a.cap]);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int idx = (i * 256 + tid) * 4, row = idx / D, col = idx % D;
    const float v = s_ve[row];
    float4 s = sr[i];
    s.x = fmaf(v, s_ke[col], s.x);
    s.y = fmaf(v, s_ke[col + 1], s.y);
    s.z = fmaf(v, s_ke[col + 2], s.z);
    s.w = fmaf(v, s_ke[col + 3], s.w);
    S4[i * 256 + tid] = s;
  }
  if (tid < D) {
    a.s_k[pair * D + tid] += s_ke[tid];
    a.s_v[pair * D + tid] += s_ve[tid];
    kr[tid] = a.k_new[pair * D + tid];
    vc[(size_t)tid * a.cap] = a.v_new[pair * D + tid];
  }
  if (tid == 0) {
    a.n_e[pair] += 1;
    a.slot_pos[pair * P + e] = p;
  }
}

template <int D>
static bool launch_commit(int G, dim3 grid, hipStream_t s, const MsArgs& a) {
  switch (G) {
    case 1: hipLaunchKernelGGL((mstream_commit_kernel<D, 1>), grid, dim3(256), 0, s, a); return true;
    case 2: hipLaunchKernelGGL((mstream_commit_kernel<D, 2>), grid, dim3(256), 0, s, a); return true;
    case 4: hipLaunchKernelGGL((mstream_commit_kernel<D, 4>), grid, dim3(256), 0, s, a); return true;
    case 8: hipLaunchKernelGGL((mstream_commit_kernel<D, 8>), grid, dim3(256), 0, s, a); return true;
    default: return false;
  }
}

struct MsWs { size_t lg, rn, total; };
static MsWs ms_ws(const kvm_mstream_desc* d) {
  const size_t pairs = (size_t)d->b * d->H_kv;
  const int G = d->H_q / d->H_kv;
  MsWs w;
  w.lg = 0;
  w.rn = align_up(pairs * G * d->P * sizeof(float), 256);
  w.total = align_up(w.rn + pairs * d->P * sizeof(float), 256);
  return w;
}

}  // namespace kvm

using namespace kvm;

extern "C" size_t kvm_moment_stream_workspace_size(const kvm_mstream_desc* d) {
  if (!d || d->b <= 0 || d->H_kv <= 0 || d->H_q <= 0 || d->P <= 0) return 0;
  return ms_ws(d).total;
}

extern "C" kvm_status kvm_moment_stream_evict(const kvm_mstream_desc* d, const void* q, const void* k_new,
                                              const void* v_new, void* Kc, void* Vc, int32_t* slot_pos,
                                              int32_t* next_pos, int32_t* n_e, float* s_k, float* s_v, float* S,
                                              int32_t* evict_slot, void* ws, size_t ws_bytes, void* stream) {
  KVM_PTR(d);
  KVM_REQUIRE(d->b > 0 && d->H_q > 0 && d->H_kv > 0, KVM_ERR_SHAPE, "b, H_q, H_kv must be positive");
  KVM_REQUIRE(d->H_q % d->H_kv == 0, KVM_ERR_SHAPE, "H_q %d not a multiple of H_kv %d", d->H_q, d->H_kv);
  const int G = d->H_q / d->H_kv;
  KVM_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, KVM_ERR_SHAPE, "group size %d not in {1,2,4,8}", G);
  KVM_REQUIRE(d->d == 64 || d->d == 128, KVM_ERR_SHAPE, "head dim %d not in {64, 128}", d->d);
  KVM_REQUIRE(d->dtype == KVM_BF16, KVM_ERR_DTYPE, "MomentKV scoring takes bf16 q, K, V (dtype %d)", d->dtype);
  KVM_REQUIRE(d->R >= 0 && d->P > d->R, KVM_ERR_RANGE, "pool %d must exceed the recent window %d", d->P, d->R);
  KVM_REQUIRE(d->cap >= d->P, KVM_ERR_RANGE, "cap %d below pool %d", d->cap, d->P);
  KVM_REQUIRE(d->cap % 8 == 0, KVM_ERR_SHAPE, "cap %d is not a multiple of 8", d->cap);
  KVM_REQUIRE((long long)d->cap * d->d * 2 < 0x7ffffff0LL, KVM_ERR_RANGE, "cap %d too large", d->cap);
  KVM_PTR_ALIGNED(q); KVM_PTR_ALIGNED(k_new); KVM_PTR_ALIGNED(v_new); KVM_PTR_ALIGNED(Kc); KVM_PTR_ALIGNED(Vc);
  KVM_PTR_ALIGNED(slot_pos); KVM_PTR_ALIGNED(next_pos); KVM_PTR_ALIGNED(n_e); KVM_PTR_ALIGNED(s_k);
  KVM_PTR_ALIGNED(s_v); KVM_PTR_ALIGNED(S); KVM_PTR_ALIGNED(evict_slot);
  const MsWs w = ms_ws(d);
  KVM_REQUIRE(ws != nullptr && ws_bytes >= w.total, KVM_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  KVM_ALIGNED(ws);
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;

  MsArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.Kc = static_cast<uint16_t*>(Kc);
  a.Vc = static_cast<uint16_t*>(Vc);
  a.slot_pos = slot_pos; a.next_pos = next_pos; a.n_e = n_e; a.s_k = s_k; a.s_v = s_v; a.S = S;
  a.evict_slot = evict_slot;
  char* base = static_cast<char*>(ws);
  a.lg = reinterpret_cast<float*>(base + w.lg);
  a.rn = reinterpret_cast<float*>(base + w.rn);
  a.H_q = d->H_q; a.H_kv = d->H_kv; a.G = d->H_q / d->H_kv; a.P = d->P; a.cap = d->cap; a.R = d->R;
  a.scale = 1.f / sqrtf((float)d->d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool wide = (long long)((d->P + 127) / 128) * d->H_kv * d->b >= 256;
  const int keys = wide ? 128 : 64;
  const dim3 sgrid((d->P + keys - 1) / keys, d->H_kv, d->b), cgrid(d->H_kv, d->b);
  if (d->d == 128) {
    if (wide) hipLaunchKernelGGL((mstream_score_kernel<128, 128>), sgrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((mstream_score_kernel<128, 64>), sgrid, dim3(256), 0, s, a);
    launch_commit<128>(a.G, cgrid, s, a);
  } else {
    if (wide) hipLaunchKernelGGL((mstream_score_kernel<64, 128>), sgrid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((mstream_score_kernel<64, 64>), sgrid, dim3(128), 0, s, a);
    launch_commit<64>(a.G, cgrid, s, a);
  }
  return check_hip(hipGetLastError(), "moment stream launch");
}
