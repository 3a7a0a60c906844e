// A7: one streaming eviction step during decode.  The pool holds P tokens per sequence
// (slots of the compact caches); each decode step scores the pool with the new token's
// indexer query, keeps the running max-pool of every pooled key, evicts the weakest token
// outside the recent window, folds it into the latent memory and hands its slot to the new
// token [IM 2.B: evicted tokens update M and b online during inference; IM 2.A: the
// indexer scores and the running max-pool].
//
// Three small kernels per step (the work is latency-bound, a few MB per step):
//   stream_proj_kernel    raw projections of the new token: W_kI x, W_g x, W_qI[h] q_c(h)
//   stream_score_kernel   QK-norms, gated per-head ReLU scores of 64 pooled keys per block,
//                         I <- max(I, score), the block's eviction candidate
//   stream_commit_kernel  the step's eviction choice and the pool bookkeeping
// followed by the rank-1 memory update of the evicted row (kvm_mem_update with row_slot).
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

constexpr int kStreamKeys = 64;   // pooled keys per score block

// grid (long_blocks + short_blocks, b), 256 threads.  Long rows (length D): d_I rows of W_kI
// and H_I rows of W_g against x, one wave per row.  Short rows (length d): the H_I * d_I
// rows of W_qI against the model query head c(h) = floor(h H_q / H_I), 16 lanes per row.
template <typename T>
__global__ __launch_bounds__(256) void stream_proj_kernel(StreamArgs a, int long_blocks) {
  constexpr int N = Vec16<T>::N;
  const int bb = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* out = a.proj + (size_t)bb * a.NP;
  if ((int)blockIdx.x < long_blocks) {
    const int row = blockIdx.x * 4 + wave;
    if (row >= a.d_I + a.H_I) return;
    const T* w = row < a.d_I ? reinterpret_cast<const T*>(a.W_kI) + (size_t)row * a.D
                             : reinterpret_cast<const T*>(a.W_g) + (size_t)(row - a.d_I) * a.D;
    const T* x = reinterpret_cast<const T*>(a.x) + (size_t)bb * a.D;
    float acc = 0.f;
    for (int k = lane * N; k < a.D; k += 64 * N) {
      float wv[N], xv[N];
      Vec16<T>::load(w + k, wv);
      Vec16<T>::load(x + k, xv);
#pragma unroll
      for (int i = 0; i < N; ++i) acc = fmaf(wv[i], xv[i], acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) out[row] = acc;
  } else {
    const int l16 = tid & 15;
    const int base = ((int)blockIdx.x - long_blocks) * 64;
    for (int r = base + (tid >> 4); r < min(base + 64, a.H_I * a.d_I); r += 16) {
      const int h = r / a.d_I;
      const int c = h * a.H_q / a.H_I;
      const T* w = reinterpret_cast<const T*>(a.W_qI) + (size_t)r * a.d;
      const T* qv = reinterpret_cast<const T*>(a.q) + ((size_t)bb * a.H_q + c) * a.d;
      float acc = 0.f;
      for (int k = l16 * N; k < a.d; k += 16 * N) {
        float wv[N], xv[N];
        Vec16<T>::load(w + k, wv);
        Vec16<T>::load(qv + k, xv);
#pragma unroll
        for (int i = 0; i < N; ++i) acc = fmaf(wv[i], xv[i], acc);
      }
      acc = group_sum<16>(acc);
      if (l16 == 0) out[a.d_I + a.H_I + r] = acc;
    }
  }
}

// grid (nsb, b), 256 threads; d_I <= 64, H_I <= 64.
__global__ __launch_bounds__(256) void stream_score_kernel(StreamArgs a) {
  const int bb = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float s_qt[64][65];          // gated, scaled, normalised queries  q~[h][i]
  __shared__ float s_key[kStreamKeys][65];
  __shared__ float s_kn[64];
  __shared__ unsigned long long s_best[4];
  __shared__ int s_bslot[4];
  const float* pr = a.proj + (size_t)bb * a.NP;
  const float inv_sqrt = rsqrtf((float)a.d_I);

  // queries: q~_h = sigmoid(W_g[h] x) / sqrt(d_I) * RMSNorm_gamma_q(q^I_h)
  for (int h = wave; h < a.H_I; h += 4) {
    const float* qi = pr + a.d_I + a.H_I + (size_t)h * a.d_I;
    const float v = lane < a.d_I ? qi[lane] : 0.f;
    const float ss = wave_sum(v * v);
    const float g = sigmoid_f(pr[a.d_I + h]);
    const float r = rsqrtf(ss / (float)a.d_I + a.eps);
    if (lane < a.d_I) s_qt[h][lane] = g * inv_sqrt * a.gamma_q[lane] * v * r;
  }
  if (wave == 0) {   // the new token's key
    const float v = lane < a.d_I ? pr[lane] : 0.f;
    const float ss = wave_sum(v * v);
    const float r = rsqrtf(ss / (float)a.d_I + a.eps);
    if (lane < a.d_I) s_kn[lane] = a.gamma_k[lane] * v * r;
  }
  // this block's pooled keys
  const int j0 = blk * kStreamKeys;
  const float* kh = a.khat + ((size_t)bb * a.P + j0) * a.d_I;
  for (int i = tid; i < kStreamKeys * a.d_I; i += 256) {
    const int k = i / a.d_I, c = i % a.d_I;
    s_key[k][c] = (j0 + k < a.P) ? kh[(size_t)k * a.d_I + c] : 0.f;
  }
  __syncthreads();

  // score of key k = tid / 4 over heads h = sub, sub + 4, ...
  const int k = tid >> 2, sub = tid & 3;
  float s = 0.f;
  for (int h = sub; h < a.H_I; h += 4) {
    float dot = 0.f;
    for (int c = 0; c < a.d_I; ++c) dot = fmaf(s_qt[h][c], s_key[k][c], dot);
    s += fmaxf(dot, 0.f);
  }
  s = group_sum<4>(s);

  const int j = j0 + k;
  const int p = a.next_pos[bb];
  unsigned long long key = ~0ull;
  if (sub == 0 && j < a.P) {
    float* Ip = a.I + (size_t)bb * a.P + j;
    const float old = *Ip;
    const float nv = (old != old || s != s) ? NAN : fmaxf(old, s);   // NaN propagates
    *Ip = nv;
    const int pos = a.slot_pos[(size_t)bb * a.P + j];
    // lowest importance first; among equal importances the higher position goes first
    if (pos <= p - a.R) key = ((unsigned long long)order_key(nv) << 32) | (uint32_t)(0x7fffffff - pos);
  }
  // block minimum of (key, slot)
  int slot = j;
  for (int off = 4; off < 64; off <<= 1) {
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
    for (int h = lane; h < a.H_I; h += 64) {
      float dot = 0.f;
      for (int c = 0; c < a.d_I; ++c) dot = fmaf(s_qt[h][c], s_kn[c], dot);
      sn += fmaxf(dot, 0.f);
    }
    sn = wave_sum(sn);
    float* ni = a.newinfo + (size_t)bb * (a.d_I + 1);
    if (lane < a.d_I) ni[lane] = s_kn[lane];
    if (lane == 0) ni[a.d_I] = sn;
  }
}

// grid (b), 64 threads: the step's eviction and the pool bookkeeping.
__global__ __launch_bounds__(64) void stream_commit_kernel(StreamArgs a) {
  const int bb = blockIdx.x, lane = threadIdx.x;
  unsigned long long key = ~0ull;
  int slot = -1;
  for (int i = lane; i < a.nsb; i += 64) {
    const unsigned long long k = a.best[(size_t)bb * a.nsb + i];
    if (k < key) { key = k; slot = a.best_slot[(size_t)bb * a.nsb + i]; }
  }
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long ok = __shfl_xor(key, off);
    const int os = __shfl_xor(slot, off);
    if (ok < key || (ok == key && os < slot)) { key = ok; slot = os; }
  }
  const int e = key == ~0ull ? -1 : slot;
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
  hipLaunchKernelGGL(stream_commit_kernel, dim3(d->b), dim3(64), 0, s, a);
  st = check_hip(hipGetLastError(), "stream kernels launch");
  if (st != KVM_OK) return st;
  // fold the evicted row (still in the caches) into M, b
  const kvm_mem_desc md{d->b, d->H_kv, d->d, 1, d->cap, d->dtype, d->lam};
  return kvm_mem_update(&md, Kc, Vc, evict_slot, M, bvec, stream);
}
