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
// Data movement: K/V rows stream from HBM with 16-byte loads; a row of d elements is
// spread over d/EPL lanes, so one wave reads 64 x 16 bytes per instruction.  Each lane
// keeps q fragments of all G heads of the group in registers, so K/V are read once for G
// query heads.  Scores are reduced across the row's lanes with DPP; the online softmax runs
// per lane group with exp2 and a pre-scaled q.  The M (or S) read-out is sliced by rows
// across the split blocks, so every block reads D/n_split rows of the d x d state.
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
  float* o;
  float* lse;
  float* part_a;    // [b, H_kv, n_split, G, D]
  float* part_lse;  // [b, H_kv, n_split, G]
  float* num;       // [b, H_kv, G, D]
  int* counters;    // [b, H_kv]
  int b, H_q, H_kv, cap, n_split, mode;
  float scale, eps;
};

static constexpr float kLog2e = 1.4426950408889634f;
static constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float xor_lane(float x, int mask) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute((__lane_id() ^ mask) << 2, __float_as_int(x)));
}

template <typename T, int D, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  constexpr int EPL = Vec16<T>::N;   // elements per lane (16 bytes)
  constexpr int LPT = D / EPL;       // lanes per token row
  constexpr int TPI = 64 / LPT;      // token rows per wave instruction
  constexpr int NT = NW * 64;
  const int c = blockIdx.x, g = blockIdx.y, bb = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPT, grp = lane / LPT;

  __shared__ float s_feat[G][D];
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_acc[NW][G][D];
  __shared__ float s_red[2][G];
  __shared__ int s_flag;

  const int len0 = a.len[bb];
  int n, app;
  if (!a.k_new) { n = len0; app = -1; }
  else if (a.append_slot) { n = len0; app = a.append_slot[bb]; }
  else { n = len0 + 1; app = len0; }
  n = min(max(n, 0), a.cap);
  if (app < 0 || app >= a.cap) app = -1;

  const int per = (n + a.n_split - 1) / a.n_split;
  const int j0 = c * per, j1 = min(n, j0 + per);

  const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)bb * a.H_q + (size_t)g * G) * D;
  const size_t cache_off = ((size_t)bb * a.H_kv + g) * (size_t)a.cap * D;
  T* Kp = reinterpret_cast<T*>(a.Kc) + cache_off;
  T* Vp = reinterpret_cast<T*>(a.Vc) + cache_off;
  const T* kn = a.k_new ? reinterpret_cast<const T*>(a.k_new) + ((size_t)bb * a.H_kv + g) * D : nullptr;
  const T* vn = a.v_new ? reinterpret_cast<const T*>(a.v_new) + ((size_t)bb * a.H_kv + g) * D : nullptr;

  // read-out features: phi(q) (memory) or q (moments), needed by the row slice below
  if (a.mode != KVM_READ_NONE) {
    for (int i = tid; i < G * D; i += NT) {
      float x = load_scalar<T>(qp + i);
      s_feat[i / D][i % D] = a.mode == KVM_READ_MEMORY ? phi_f(x) : x;
    }
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

  for (int j = j0 + wave * TPI + grp; j < j1; j += NW * TPI) {
    const bool is_new = (j == app);
    const T* kr = is_new ? kn : Kp + (size_t)j * D;
    const T* vr = is_new ? vn : Vp + (size_t)j * D;
    const uint4 kraw = *reinterpret_cast<const uint4*>(kr + sub * EPL);
    const uint4 vraw = *reinterpret_cast<const uint4*>(vr + sub * EPL);
    if (is_new) {
      *reinterpret_cast<uint4*>(Kp + (size_t)j * D + sub * EPL) = kraw;
      *reinterpret_cast<uint4*>(Vp + (size_t)j * D + sub * EPL) = vraw;
    }
    float kf[EPL], vf[EPL];
    Vec16<T>::unpack(kraw, kf);
    Vec16<T>::unpack(vraw, vf);
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

  // merge the TPI lane groups of the wave (lanes sub, sub+LPT, ...)
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

  // block state -> workspace
  const size_t pair = (size_t)bb * a.H_kv + g;
  float* pa = a.part_a + (pair * a.n_split + c) * (size_t)(G * D);
  for (int i = tid; i < G * D; i += NT) {
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

  // read-out numerator rows of this block's slice: num[h][r] = sum_k Mat[r][k] feat_h[k]
  if (a.mode != KVM_READ_NONE) {
    const float* Mat = (a.mode == KVM_READ_MEMORY ? a.M : a.S) + pair * (size_t)(D * D);
    const int rps = (D + a.n_split - 1) / a.n_split;
    const int r0 = c * rps, r1 = min(D, r0 + rps);
    constexpr int CPL = D / 64;  // columns per lane
    for (int r = r0 + wave; r < r1; r += NW) {
      float mr[CPL];
#pragma unroll
      for (int k = 0; k < CPL; ++k) mr[k] = Mat[(size_t)r * D + lane * CPL + k];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = 0.f;
#pragma unroll
        for (int k = 0; k < CPL; ++k) x = fmaf(mr[k], s_feat[h][lane * CPL + k], x);
        x = wave_sum(x);
        if (lane == 0) a.num[(pair * G + h) * D + r] = x;
      }
    }
  }

  if (!last_block_ticket(a.counters + pair, a.n_split, &s_flag)) return;

  // ---------------------------------------------------------------- last block: merge
  // per-head scalars of the read-out
  if (a.mode == KVM_READ_MEMORY) {
    for (int h = wave; h < G; h += NW) {
      float den = 0.f, gl = 0.f;
      const T* wg = reinterpret_cast<const T*>(a.w_g) + (size_t)(g * G + h) * D;
      for (int k = lane; k < D; k += 64) {
        den = fmaf(a.bvec[pair * D + k], s_feat[h][k], den);
        gl = fmaf(load_scalar<T>(wg + k), load_scalar<T>(qp + h * D + k), gl);
      }
      den = wave_sum(den);
      gl = wave_sum(gl);
      if (lane == 0) { s_red[0][h] = den + a.eps; s_red[1][h] = sigmoid_f(gl); }
    }
  } else if (a.mode == KVM_READ_MOMENTS) {
    for (int h = wave; h < G; h += NW) {
      float sq = 0.f;
      for (int k = lane; k < D; k += 64) sq = fmaf(a.s_k[pair * D + k], s_feat[h][k], sq);
      sq = wave_sum(sq);
      if (lane == 0) s_red[0][h] = sq;
    }
  }
  __syncthreads();

  const float* pl = a.part_lse + pair * a.n_split * G;
  const float* pa0 = a.part_a + pair * a.n_split * (size_t)(G * D);
  const int ne = a.mode == KVM_READ_MOMENTS ? a.n_e[pair] : 0;
  for (int i = tid; i < G * D; i += NT) {
    const int h = i / D, dd = i % D;
    float mx = -INFINITY;
    for (int cc = 0; cc < a.n_split; ++cc) mx = fmaxf(mx, pl[cc * G + h]);
    float lse = -INFINITY, o = 0.f;
    if (mx != -INFINITY) {
      float Z = 0.f;
      for (int cc = 0; cc < a.n_split; ++cc) Z += __expf(pl[cc * G + h] - mx);
      lse = mx + __logf(Z);
      for (int cc = 0; cc < a.n_split; ++cc) {
        const float w = __expf(pl[cc * G + h] - lse);
        o = fmaf(w, pa0[(size_t)cc * G * D + i], o);
      }
    }
    if (a.mode == KVM_READ_MEMORY) {
      o = fmaf(s_red[1][h], a.num[(pair * G + h) * D + dd] / s_red[0][h], o);
    } else if (a.mode == KVM_READ_MOMENTS && ne > 0) {
      const float inv = 1.f / (float)ne;
      const float sq = s_red[0][h];
      const float sv = a.s_v[pair * D + dd];
      const float fE = sv * inv + a.scale * (a.num[(pair * G + h) * D + dd] - sv * sq * inv) * inv;
      const float logZ = __logf((float)ne) + a.scale * sq * inv;
      const float w = sigmoid_f(lse - logZ);
      o = w * o + (1.f - w) * fE;
    }
    a.o[((size_t)bb * a.H_q + g * G + h) * D + dd] = o;
    if (a.lse && dd == 0) a.lse[(size_t)bb * a.H_q + g * G + h] = lse;
  }
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
  size_t a, lse, num, cnt, total;
};
static DecodeWs decode_ws(const kvm_decode_desc* d, int ns) {
  const int G = d->H_q / d->H_kv;
  const size_t pairs = (size_t)d->b * d->H_kv;
  DecodeWs w;
  w.cnt = 0;
  w.a = kCounterBytes;
  w.lse = align_up(w.a + pairs * ns * G * d->d * sizeof(float), 256);
  w.num = align_up(w.lse + pairs * ns * G * sizeof(float), 256);
  w.total = align_up(w.num + pairs * G * d->d * sizeof(float), 256);
  return w;
}

template <typename T, int D, int G>
static void launch_decode(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.n_split, a.H_kv, a.b);
  hipLaunchKernelGGL((decode_kernel<T, D, G, 4>), grid, dim3(256), 0, st, a);
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
  KVM_REQUIRE(d->d == 64 || d->d == 128, KVM_ERR_SHAPE, "head dim %d not in {64, 128}", d->d);
  KVM_REQUIRE(d->H_q % d->H_kv == 0, KVM_ERR_SHAPE, "H_q %% H_kv != 0");
  const int G = d->H_q / d->H_kv;
  KVM_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, KVM_ERR_SHAPE, "group size %d not in {1,2,4,8}", G);
  KVM_REQUIRE(d->dtype == KVM_F32 || d->dtype == KVM_BF16, KVM_ERR_DTYPE, "dtype %d", d->dtype);
  KVM_REQUIRE(d->mode >= KVM_READ_NONE && d->mode <= KVM_READ_MOMENTS, KVM_ERR_RANGE, "mode %d", d->mode);
  KVM_REQUIRE(d->n_split >= 0 && d->n_split <= 256, KVM_ERR_RANGE, "n_split %d", d->n_split);
  KVM_PTR_ALIGNED(q); KVM_PTR_ALIGNED(Kc); KVM_PTR_ALIGNED(Vc); KVM_PTR_ALIGNED(len); KVM_PTR_ALIGNED(o);
  KVM_REQUIRE((k_new == nullptr) == (v_new == nullptr), KVM_ERR_NULL, "k_new and v_new must both be given or both NULL");
  KVM_REQUIRE(append_slot == nullptr || k_new != nullptr, KVM_ERR_NULL, "append_slot needs k_new");
  KVM_OPT_ALIGNED(k_new); KVM_OPT_ALIGNED(v_new); KVM_OPT_ALIGNED(lse);
  if (d->mode == KVM_READ_MEMORY) { KVM_PTR_ALIGNED(M); KVM_PTR_ALIGNED(bvec); KVM_PTR_ALIGNED(w_g); }
  if (d->mode == KVM_READ_MOMENTS) {
    KVM_PTR_ALIGNED(n_e); KVM_PTR_ALIGNED(s_k); KVM_PTR_ALIGNED(s_v); KVM_PTR_ALIGNED(S);
  }
  KVM_REQUIRE((size_t)d->b * d->H_kv <= (size_t)kMaxCounters, KVM_ERR_SHAPE, "b * H_kv exceeds %d", kMaxCounters);
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
  char* base = static_cast<char*>(ws);
  a.part_a = reinterpret_cast<float*>(base + w.a);
  a.part_lse = reinterpret_cast<float*>(base + w.lse);
  a.num = reinterpret_cast<float*>(base + w.num);
  a.counters = reinterpret_cast<int*>(base + w.cnt);
  a.b = d->b; a.H_q = d->H_q; a.H_kv = d->H_kv; a.cap = d->cap; a.n_split = ns; a.mode = d->mode;
  a.scale = d->scale; a.eps = d->eps;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool ok;
  if (d->dtype == KVM_BF16)
    ok = d->d == 128 ? dispatch_g<uint16_t, 128>(G, a, s) : dispatch_g<uint16_t, 64>(G, a, s);
  else
    ok = d->d == 128 ? dispatch_g<float, 128>(G, a, s) : dispatch_g<float, 64>(G, a, s);
  if (!ok) return set_error(KVM_ERR_SHAPE, "unsupported group size");
  return check_hip(hipGetLastError(), "decode_kernel launch");
}

extern "C" kvm_status kvm_len_add(int32_t* len, int32_t b, int32_t delta, void* stream) {
  KVM_PTR_ALIGNED(len);
  KVM_REQUIRE(b > 0, KVM_ERR_SHAPE, "b must be positive");
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;
  hipLaunchKernelGGL(len_add_kernel, dim3((b + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), len, b, delta);
  return check_hip(hipGetLastError(), "len_add launch");
}
