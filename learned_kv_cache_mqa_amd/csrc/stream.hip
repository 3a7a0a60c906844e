// A7: one streaming eviction step during decode.  The pool holds P tokens per sequence
// (slots of the compact caches); each decode step scores the pool with the new token's
// indexer query, keeps the running max-pool of every pooled key, evicts the weakest token
// outside the recent window, folds it into the latent memory and hands its slot to the new
// token [IM 2.B: evicted tokens update M and b online during inference; IM 2.A: the
// indexer scores and the running max-pool].
//
// Three small kernels per step (the work is latency-bound, a few MB per step, so each kernel
// issues all of its global loads before its first dependent use):
//   stream_proj_kernel    raw projections of the new token: W_kI x, W_g x, W_qI[h] q_c(h)
//   stream_score_kernel   QK-norms, gated per-head ReLU scores of 16 pooled keys per block,
//                         I <- max(I, score), the block's eviction candidate
//   stream_commit_kernel  the step's eviction choice, the pool bookkeeping and the rank-1
//                         memory update of the evicted row, read from the caches before the
//                         decode's append overwrites its slot
#include "common.hpp"

namespace kvm {

struct StreamArgs {
  const void* x;       // [b, D]
  const void* q;       // [b, H_q, d]
  const void* W_kI;    // [d_I, D]
  const float* gamma_k;
  const void* W_qI;    // [H_I, d_I, d]
  const float* gamma_q;
  const void* W_g;     // [H_I, D]
  float* khat;         // [b, P, d_I]
  float* I;            // [b, P]
  int32_t* slot_pos;   // [b, P]
  int32_t* next_pos;   // [b]
  int32_t* evict_slot; // [b]
  float* proj;         // ws [b, NP]
  unsigned long long* best;  // ws [b, nsb]
  int* best_slot;      // ws [b, nsb]
  float* newinfo;      // ws [b, d_I + 1]: k_hat of the new token, its self-score
  int D, H_q, d, H_I, d_I, P, R, nsb, NP;
  float eps;
};

constexpr int kStreamKeys = 16;                  // pooled keys per score block
constexpr int kThreadsPerKey = 256 / kStreamKeys;  // lanes sharing one key's heads
constexpr int kKeyDims = 64 / kThreadsPerKey;      // key dims each lane loads
constexpr int kRowPitch = 68;     // LDS row pitch (floats) of queries and keys: 16-byte aligned rows

__device__ __forceinline__ float loadf(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// grid (long_blocks + short_blocks, b), 256 threads.  Long rows (length D): d_I rows of W_kI
// and H_I rows of W_g against x, one wave per row.  Short rows (length d <= 128): the
// H_I * d_I rows of W_qI against the model query head c(h) = floor(h H_q / H_I), 16 lanes per
// row, 64 rows per block.  Loads go through buffer resources (zeros past the end), so every
// load of a lane is issued before the first product.
template <typename T>
__global__ __launch_bounds__(256) void stream_proj_kernel(StreamArgs a, int long_blocks) {
  constexpr int N = Vec16<T>::N;
  constexpr int TB = (int)sizeof(T);
  // the wave index through readfirstlane: buffer resources built from it stay scalar (a
  // per-lane value there turns every load into a loop over the distinct lane values)
  const int bb = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* out = a.proj + (size_t)bb * a.NP;
  if ((int)blockIdx.x < long_blocks) {
    const int row = blockIdx.x * 4 + wave;
    if (row >= a.d_I + a.H_I) return;
    const T* w = row < a.d_I ? reinterpret_cast<const T*>(a.W_kI) + (size_t)row * a.D
                             : reinterpret_cast<const T*>(a.W_g) + (size_t)(row - a.d_I) * a.D;
    const auto rw = make_rsrc(w, a.D * TB);
    const auto rx = make_rsrc(reinterpret_cast<const T*>(a.x) + (size_t)bb * a.D, a.D * TB);
    constexpr int U = 8;
    float acc = 0.f;
    for (int k0 = 0; k0 < a.D; k0 += U * 64 * N) {
      uint4 wr[U], xr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int off = (k0 + (u * 64 + lane) * N) * TB;
        wr[u] = load16(rw, off);
        xr[u] = load16(rx, off);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float wv[N], xv[N];
        Vec16<T>::unpack(wr[u], wv);
        Vec16<T>::unpack(xr[u], xv);
#pragma unroll
        for (int i = 0; i < N; ++i) acc = fmaf(wv[i], xv[i], acc);
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) out[row] = acc;
  } else {
    constexpr int CH = (128 + 16 * N - 1) / (16 * N);   // 16-byte chunks per lane and row (d <= 128)
    const int l16 = tid & 15, grp = tid >> 4;
    const int base = ((int)blockIdx.x - long_blocks) * 64;
    const int nrows = a.H_I * a.d_I;
    const auto rw = make_rsrc(a.W_qI, nrows * a.d * TB);
    const auto rq = make_rsrc(reinterpret_cast<const T*>(a.q) + (size_t)bb * a.H_q * a.d, a.H_q * a.d * TB);
    uint4 wr[4][CH], qr[4][CH];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = base + grp + 16 * u;
      const int c = (r / a.d_I) * a.H_q / a.H_I;
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        const int k = (ch * 16 + l16) * N;
        wr[u][ch] = load16(rw, (r * a.d + k) * TB);
        qr[u][ch] = load16(rq, (c * a.d + k) * TB);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = base + grp + 16 * u;
      float acc = 0.f;
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        if ((ch * 16 + l16) * N < a.d) {
          float wv[N], xv[N];
          Vec16<T>::unpack(wr[u][ch], wv);
          Vec16<T>::unpack(qr[u][ch], xv);
#pragma unroll
          for (int i = 0; i < N; ++i) acc = fmaf(wv[i], xv[i], acc);
        }
      }
      acc = group_sum<16>(acc);
      if (l16 == 0 && r < min(base + 64, nrows)) out[a.d_I + a.H_I + r] = acc;
    }
  }
}

// grid (nsb, b), 256 threads; d_I <= 64, H_I <= 64.  Every global load of the block (the
// projections, the block's 16 pooled keys, their importances and positions) is issued at
// the start; queries and keys are then staged in LDS, zero past d_I.
__global__ __launch_bounds__(256) void stream_score_kernel(StreamArgs a) {
  const int bb = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ __align__(16) float s_q[64 * kRowPitch];            // q~[h][c]
  __shared__ __align__(16) float s_key[kStreamKeys * kRowPitch];  // pooled keys [k][c]
  __shared__ __align__(16) float s_kn[64];                        // the new token's key
  __shared__ unsigned long long s_best[4];
  __shared__ int s_bslot[4];
  const int dI = a.d_I, HI = a.H_I;
  const int j0 = blk * kStreamKeys, nk = min(kStreamKeys, a.P - j0);

  const auto rp = make_rsrc(a.proj + (size_t)bb * a.NP, a.NP * 4);
  const auto rgq = make_rsrc(a.gamma_q, dI * 4);
  // queries: heads hq and hq + 32, dims c8 .. c8 + 7
  const int hq = tid >> 3, c8 = (tid & 7) * 8;
  float qv[2][8], gq[8], gate[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int h = hq + 32 * u;
    gate[u] = loadf(rp, (dI + h) * 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[u][i] = loadf(rp, (dI + HI + h * dI + c8 + i) * 4);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) gq[i] = loadf(rgq, (c8 + i) * 4);
  // the new token's key, dim = lane
  const float kn = loadf(rp, lane * 4);
  const float gk = loadf(make_rsrc(a.gamma_k, dI * 4), lane * 4);
  // pooled key k, dims kKeyDims sub .. kKeyDims (sub + 1) - 1
  const int k = tid / kThreadsPerKey, sub = tid % kThreadsPerKey;
  const auto rk = make_rsrc(a.khat + ((size_t)bb * a.P + j0) * dI, nk * dI * 4);
  float kv[kKeyDims];
#pragma unroll
  for (int i = 0; i < kKeyDims; ++i) kv[i] = loadf(rk, (k * dI + sub * kKeyDims + i) * 4);
  const float Iold = loadf(make_rsrc(a.I + (size_t)bb * a.P + j0, nk * 4), k * 4);
  const int pos = (int)__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.slot_pos + (size_t)bb * a.P + j0, nk * 4),
                                                            k * 4, 0, 0);
  const int p = (int)__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.next_pos + bb, 4), 0, 0, 0);

  // q~_h = sigmoid(W_g[h] x) / sqrt(d_I) * RMSNorm_gamma_q(q^I_h)
  const float inv_sqrt = rsqrtf((float)dI);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qv[u][i] = c8 + i < dI ? qv[u][i] : 0.f;
      ss = fmaf(qv[u][i], qv[u][i], ss);
    }
    ss = group_sum<8>(ss);
    const float r = rsqrtf(ss / (float)dI + a.eps);
    const float g = sigmoid_f(gate[u]) * inv_sqrt;
    float* dst = s_q + (hq + 32 * u) * kRowPitch + c8;
#pragma unroll
    for (int i = 0; i < 8; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(g * gq[i] * qv[u][i] * r, g * gq[i + 1] * qv[u][i + 1] * r,
                                                        g * gq[i + 2] * qv[u][i + 2] * r,
                                                        g * gq[i + 3] * qv[u][i + 3] * r);
  }
  {
    const int c0 = sub * kKeyDims;
    float* dst = s_key + k * kRowPitch + c0;
#pragma unroll
    for (int i = 0; i < kKeyDims; i += 4) {
      float4 t;
      t.x = c0 + i < dI ? kv[i] : 0.f;
      t.y = c0 + i + 1 < dI ? kv[i + 1] : 0.f;
      t.z = c0 + i + 2 < dI ? kv[i + 2] : 0.f;
      t.w = c0 + i + 3 < dI ? kv[i + 3] : 0.f;
      *reinterpret_cast<float4*>(dst + i) = t;
    }
  }
  if (wave == 0) {   // k_hat_new = RMSNorm_gamma_k(W_kI x)
    const float v = lane < dI ? kn : 0.f;
    const float ss = wave_sum(v * v);
    const float r = rsqrtf(ss / (float)dI + a.eps);
    s_kn[lane] = gk * v * r;
  }
  __syncthreads();

  // score of key k over heads h = sub, sub + kThreadsPerKey, ...: the key from registers,
  // the queries broadcast from LDS
  float kr[64];
#pragma unroll
  for (int c = 0; c < 64; c += 4) {
    const float4 t = *reinterpret_cast<const float4*>(s_key + k * kRowPitch + c);
    kr[c] = t.x; kr[c + 1] = t.y; kr[c + 2] = t.z; kr[c + 3] = t.w;
  }
  float s = 0.f;
  for (int h = sub; h < HI; h += kThreadsPerKey) {
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < 64; c += 4) {
      const float4 q = *reinterpret_cast<const float4*>(s_q + h * kRowPitch + c);
      dot = fmaf(q.x, kr[c], dot);
      dot = fmaf(q.y, kr[c + 1], dot);
      dot = fmaf(q.z, kr[c + 2], dot);
      dot = fmaf(q.w, kr[c + 3], dot);
    }
    s += fmaxf(dot, 0.f);
  }
  s = group_sum<kThreadsPerKey>(s);

  const int j = j0 + k;
  unsigned long long key = ~0ull;
  if (sub == 0 && k < nk) {
    const float nv = (Iold != Iold || s != s) ? NAN : fmaxf(Iold, s);   // NaN propagates
    a.I[(size_t)bb * a.P + j] = nv;
    // lowest importance first; among equal importances the higher position goes first
    if (pos <= p - a.R) key = ((unsigned long long)order_key(nv) << 32) | (uint32_t)(0x7fffffff - pos);
  }
  // block minimum of (key, slot)
  int slot = j;
  for (int off = kThreadsPerKey; off < 64; off <<= 1) {
    const unsigned long long ok = __shfl_xor(key, off);
    const int os = __shfl_xor(slot, off);
    if (ok < key) { key = ok; slot = os; }
  }
  if (lane == 0) { s_best[wave] = key; s_bslot[wave] = slot; }
  __syncthreads();
  if (tid == 0) {
    unsigned long long bk = s_best[0];
    int bs = s_bslot[0];
    for (int w = 1; w < 4; ++w)
      if (s_best[w] < bk) { bk = s_best[w]; bs = s_bslot[w]; }
    a.best[(size_t)bb * a.nsb + blk] = bk;
    a.best_slot[(size_t)bb * a.nsb + blk] = bs;
  }
  if (blk == 0 && wave == 0) {   // the new token's own score and key
    float sn = 0.f;
    if (lane < HI) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < 64; c += 4) {
        const float4 q = *reinterpret_cast<const float4*>(s_q + lane * kRowPitch + c);
        const float4 kk = *reinterpret_cast<const float4*>(s_kn + c);
        dot = fmaf(q.x, kk.x, dot);
        dot = fmaf(q.y, kk.y, dot);
        dot = fmaf(q.z, kk.z, dot);
        dot = fmaf(q.w, kk.w, dot);
      }
      sn = fmaxf(dot, 0.f);
    }
    sn = wave_sum(sn);
    float* ni = a.newinfo + (size_t)bb * (a.d_I + 1);
    if (lane < a.d_I) ni[lane] = s_kn[lane];
    if (lane == 0) ni[a.d_I] = sn;
  }
}

struct CommitMem {
  const void* Kc;   // [b, H_kv, cap, d]
  const void* Vc;   // [b, H_kv, d, cap]
  float* M;         // [b, H_kv, d, d]
  float* bvec;      // [b, H_kv, d]
  int H_kv, cap;
  float lam;
};

// grid (d * d / 1024, H_kv, b), 256 threads.  Every block reduces the score blocks'
// candidates to the step's eviction e (the same in every block).  Block (0, 0) does the
// pool bookkeeping; every block folds the evicted row into its 1024 elements of M,
// M <- lam M + v_e phi(k_e)^T, and block x == 0 also updates b <- lam b + phi(k_e).
template <typename T, int D>
__global__ __launch_bounds__(256) void stream_commit_kernel(StreamArgs a, CommitMem m) {
  const int bb = blockIdx.z, g = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const size_t pair = (size_t)bb * m.H_kv + g;
  const int e0 = (blockIdx.x * 256 + tid) * 4, row = e0 / D, col = e0 % D;
  float4* Mp = reinterpret_cast<float4*>(m.M + pair * D * D + e0);
  const float4 mo = *Mp;   // independent of the choice
  const auto rb = make_rsrc(m.bvec + pair * D, blockIdx.x == 0 ? D * 4 : 0);
  const float bo = loadf(rb, tid * 4);

  unsigned long long key = ~0ull;
  int slot = -1;
  for (int i = lane; i < a.nsb; i += 64) {
    const unsigned long long kk = a.best[(size_t)bb * a.nsb + i];
    const int ks = a.best_slot[(size_t)bb * a.nsb + i];
    if (kk < key) { key = kk; slot = ks; }
  }
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long ok = __shfl_xor(key, off);
    const int os = __shfl_xor(slot, off);
    if (ok < key || (ok == key && os < slot)) { key = ok; slot = os; }
  }
  const int e = key == ~0ull ? -1 : slot;
  if (blockIdx.x == 0 && g == 0 && tid < 64) {
    const int p = a.next_pos[bb];
    const float* ni = a.newinfo + (size_t)bb * (a.d_I + 1);
    if (e >= 0 && lane < a.d_I) a.khat[((size_t)bb * a.P + e) * a.d_I + lane] = ni[lane];
    if (lane == 0) {
      a.evict_slot[bb] = e;
      if (e >= 0) {
        a.slot_pos[(size_t)bb * a.P + e] = p;
        a.I[(size_t)bb * a.P + e] = ni[a.d_I];
      }
      a.next_pos[bb] = p + 1;
    }
  }
  if (e < 0) return;   // nothing evicted: M and b stay
  const T* kp = reinterpret_cast<const T*>(m.Kc) + (pair * m.cap + e) * D;
  const float v = load_scalar<T>(reinterpret_cast<const T*>(m.Vc) + (pair * D + row) * m.cap + e);
  float u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = v * phi_f(load_scalar<T>(kp + col + i));
  *Mp = make_float4(fmaf(m.lam, mo.x, u[0]), fmaf(m.lam, mo.y, u[1]), fmaf(m.lam, mo.z, u[2]),
                    fmaf(m.lam, mo.w, u[3]));
  if (blockIdx.x == 0 && tid < D) m.bvec[pair * D + tid] = fmaf(m.lam, bo, phi_f(load_scalar<T>(kp + tid)));
}

struct StreamWs { size_t proj, best, bslot, info, total; };
static StreamWs stream_ws(const kvm_stream_desc* d) {
  const int nsb = (d->P + kStreamKeys - 1) / kStreamKeys;
  const size_t NP = (size_t)d->d_I + d->H_I + (size_t)d->H_I * d->d_I;
  StreamWs w;
  w.proj = 0;
  w.best = align_up(w.proj + (size_t)d->b * NP * sizeof(float), 256);
  w.bslot = align_up(w.best + (size_t)d->b * nsb * sizeof(unsigned long long), 256);
  w.info = align_up(w.bslot + (size_t)d->b * nsb * sizeof(int), 256);
  w.total = align_up(w.info + (size_t)d->b * (d->d_I + 1) * sizeof(float), 256);
  return w;
}

}  // namespace kvm

using namespace kvm;

extern "C" size_t kvm_stream_workspace_size(const kvm_stream_desc* d) {
  if (!d || d->b <= 0 || d->P <= 0 || d->H_I <= 0 || d->d_I <= 0) return 0;
  return stream_ws(d).total;
}

extern "C" kvm_status kvm_stream_evict(const kvm_stream_desc* d, const void* x_new, const void* q_new,
                                       const void* W_kI, const float* gamma_k, const void* W_qI,
                                       const float* gamma_q, const void* W_g, float* khat_pool, float* I_pool,
                                       int32_t* slot_pos, int32_t* next_pos, const void* Kc, const void* Vc,
                                       float* M, float* bvec, int32_t* evict_slot, void* ws, size_t ws_bytes,
                                       void* stream) {
  KVM_PTR(d);
  KVM_REQUIRE(d->b > 0 && d->D > 0 && d->H_q > 0 && d->H_kv > 0, KVM_ERR_SHAPE, "b, D, H_q, H_kv must be positive");
  KVM_REQUIRE(d->H_q % d->H_kv == 0, KVM_ERR_SHAPE, "H_q %d not a multiple of H_kv %d", d->H_q, d->H_kv);
  KVM_REQUIRE(d->d == 64 || d->d == 128, KVM_ERR_SHAPE, "head dim %d not in {64, 128}", d->d);
  KVM_REQUIRE(d->d_I >= 1 && d->d_I <= 64, KVM_ERR_SHAPE, "indexer dim %d not in [1, 64]", d->d_I);
  KVM_REQUIRE(d->H_I >= 1 && d->H_I <= 64, KVM_ERR_SHAPE, "indexer heads %d not in [1, 64]", d->H_I);
  KVM_REQUIRE(d->D % 8 == 0, KVM_ERR_SHAPE, "D %d not a multiple of 8", d->D);
  KVM_REQUIRE(d->dtype == KVM_F32 || d->dtype == KVM_BF16, KVM_ERR_DTYPE, "dtype %d", d->dtype);
  KVM_REQUIRE(d->R >= 0 && d->P > d->R, KVM_ERR_RANGE, "pool %d must exceed the recent window %d", d->P, d->R);
  KVM_REQUIRE(d->cap >= d->P, KVM_ERR_RANGE, "cap %d below pool %d", d->cap, d->P);
  KVM_REQUIRE(d->lam >= 0.f && d->lam <= 1.f, KVM_ERR_RANGE, "lam %g outside [0, 1]", d->lam);
  KVM_PTR_ALIGNED(x_new); KVM_PTR_ALIGNED(q_new); KVM_PTR_ALIGNED(W_kI); KVM_PTR_ALIGNED(gamma_k);
  KVM_PTR_ALIGNED(W_qI); KVM_PTR_ALIGNED(gamma_q); KVM_PTR_ALIGNED(W_g); KVM_PTR_ALIGNED(khat_pool);
  KVM_PTR_ALIGNED(I_pool); KVM_PTR_ALIGNED(slot_pos); KVM_PTR_ALIGNED(next_pos); KVM_PTR_ALIGNED(Kc);
  KVM_PTR_ALIGNED(Vc); KVM_PTR_ALIGNED(M); KVM_PTR_ALIGNED(bvec); KVM_PTR_ALIGNED(evict_slot);
  const StreamWs w = stream_ws(d);
  KVM_REQUIRE(ws != nullptr && ws_bytes >= w.total, KVM_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  KVM_ALIGNED(ws);
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;

  StreamArgs a{};
  a.x = x_new; a.q = q_new; a.W_kI = W_kI; a.gamma_k = gamma_k; a.W_qI = W_qI; a.gamma_q = gamma_q; a.W_g = W_g;
  a.khat = khat_pool; a.I = I_pool; a.slot_pos = slot_pos; a.next_pos = next_pos; a.evict_slot = evict_slot;
  char* base = static_cast<char*>(ws);
  a.proj = reinterpret_cast<float*>(base + w.proj);
  a.best = reinterpret_cast<unsigned long long*>(base + w.best);
  a.best_slot = reinterpret_cast<int*>(base + w.bslot);
  a.newinfo = reinterpret_cast<float*>(base + w.info);
  a.D = d->D; a.H_q = d->H_q; a.d = d->d; a.H_I = d->H_I; a.d_I = d->d_I; a.P = d->P; a.R = d->R;
  a.nsb = (d->P + kStreamKeys - 1) / kStreamKeys;
  a.NP = d->d_I + d->H_I + d->H_I * d->d_I;
  a.eps = d->eps_rms;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int long_blocks = (d->d_I + d->H_I + 3) / 4;
  const int short_blocks = (d->H_I * d->d_I + 63) / 64;
  const dim3 pgrid(long_blocks + short_blocks, d->b);
  if (d->dtype == KVM_BF16) hipLaunchKernelGGL(stream_proj_kernel<uint16_t>, pgrid, dim3(256), 0, s, a, long_blocks);
  else hipLaunchKernelGGL(stream_proj_kernel<float>, pgrid, dim3(256), 0, s, a, long_blocks);
  hipLaunchKernelGGL(stream_score_kernel, dim3(a.nsb, d->b), dim3(256), 0, s, a);
  const CommitMem m{Kc, Vc, M, bvec, d->H_kv, d->cap, d->lam};
  const dim3 cgrid(d->d * d->d / 1024, d->H_kv, d->b);
  if (d->dtype == KVM_BF16) {
    if (d->d == 128) hipLaunchKernelGGL((stream_commit_kernel<uint16_t, 128>), cgrid, dim3(256), 0, s, a, m);
    else hipLaunchKernelGGL((stream_commit_kernel<uint16_t, 64>), cgrid, dim3(256), 0, s, a, m);
  } else {
    if (d->d == 128) hipLaunchKernelGGL((stream_commit_kernel<float, 128>), cgrid, dim3(256), 0, s, a, m);
    else hipLaunchKernelGGL((stream_commit_kernel<float, 64>), cgrid, dim3(256), 0, s, a, m);
  }
  return check_hip(hipGetLastError(), "stream kernels launch");
}
