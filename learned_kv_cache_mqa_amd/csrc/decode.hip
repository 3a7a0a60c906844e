// A8 + A9 (+ V3): split-K decode attention over the retained cache, merged with the
// online-softmax identity, plus the latent-memory (or moment) read-out.
//
// Attention states: a state (a_c, lse_c) per query head of the GQA group is the attention
// output over a set of slots and the log of its normaliser [ASM, Method: attention state
// (a, Z)].  States over disjoint sets merge in a fixed order: lse = log sum exp(lse_c),
// a = sum exp(lse_c - lse) a_c [ASM, Method: online-softmax merge].  The read-out adds
// o = a + g(q) m(q) with m(q) = M phi(q) / (b . phi(q) + eps), g(q) = sigmoid(w_g . q)
// [IM 2.B, output], or mixes with the moment estimate [MKV 2, 4].
//
// Cache layout: Kc [b, H_kv, cap, d] (slot-major), Vc [b, H_kv, d, cap] (dim-major).
//
// Two kernels:
//  attention  grid (n_split, H_kv, b): each block reduces the cached slots of one slot range
//             of one (sequence, KV head) to a state per query head.  The slot that takes
//             the new token is skipped (its cached contents are stale); the block writes its
//             share of the new token's dims into that slot.  The block also computes its
//             slice of the read-out rows M phi(q).
//  merge      grid (d / 32, H_kv, b): thread (h, dim) merges the block states in chunk order,
//             then the new token's own state (a = v_new, lse = scale q . k_new), and adds the
//             read-out.  The kernel boundary makes the block states visible across the
//             chip's XCDs; a per-block release/acquire handshake inside one kernel would cost
//             an L2 write-back per block on this part.
//
// bf16, d = 128 (matrix-core path): a wave takes 32-slot tiles.  The scores run on
// v_mfma_f32_16x16x32_bf16 as S^T = K q^T: K rows (read straight from HBM, 4 lanes x 16
// bytes = 64 contiguous bytes of a row per instruction) are the A operand, in a slot order
// chosen so that each lane ends up holding one head's scores for 8 consecutive slots.  That
// is the A-operand layout of P V, which runs on the same instruction with P (bf16 hi + lo,
// 16-bit accurate) and the dim-major V cache as the B operand (each lane reads 8 consecutive
// slots of one dim, 16 contiguous bytes).  So P stays in registers, and the softmax needs a
// cross-lane step only for the tile max.  Every K/V load is a raw buffer load: lanes whose
// slots lie past the block's range use an offset past the buffer's end and read zeros
// without touching memory, so no load sits behind a branch and each wait is for exactly the
// tile being consumed.  K/V bytes are read once for all G heads.  Other shapes (fp32,
// d = 64) use an FMA path.
#include <mutex>

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
  int b, H_q, H_kv, cap, n_split, mode;
  float scale, eps;
  const void* q_mem;  // the query the memory read-out addresses M with (q unless projected)
};

static constexpr float kLog2e = 1.4426950408889634f;
static constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float xor_lane(float x, int mask) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute((__lane_id() ^ mask) << 2, __float_as_int(x)));
}

struct Span {
  int n, app, j0, j1;
};

// The kernel arguments a kernel's first loads depend on, forced into scalar registers at one
// point: their scalar loads then go out in one round.  Left to itself the compiler issues them
// in two or three dependent rounds (a batch, a wait, the next batch), each a full
// kernel-argument latency ahead of the first data load.
__device__ __forceinline__ void args_early(const DecodeArgs& a) {
  asm volatile("" ::"s"(a.q), "s"(a.k_new), "s"(a.v_new), "s"(a.append_slot), "s"(a.Kc), "s"(a.Vc), "s"(a.len),
               "s"(a.rmat), "s"(a.b), "s"(a.H_q), "s"(a.H_kv), "s"(a.cap), "s"(a.n_split), "s"(a.mode));
}
__device__ __forceinline__ void args_merge(const DecodeArgs& a) {
  asm volatile("" ::"s"(a.q), "s"(a.k_new), "s"(a.v_new), "s"(a.append_slot), "s"(a.len), "s"(a.bvec), "s"(a.w_g),
               "s"(a.n_e), "s"(a.s_k), "s"(a.s_v), "s"(a.o), "s"(a.lse), "s"(a.part_a), "s"(a.part_lse), "s"(a.num),
               "s"(a.q_mem), "s"(a.H_q), "s"(a.H_kv), "s"(a.cap), "s"(a.n_split), "s"(a.mode), "s"(a.scale),
               "s"(a.eps));
}

// The sequence's cache length and append slot (read once, early: their latency overlaps
// the loads that do not depend on them).
struct SeqLen {
  int len0, aslot;
};
// Read as vector loads: they count in order with the other vector loads, so waiting for
// them does not wait for loads issued after (scalar loads return out of order, and a wait
// for any later kernel argument would wait for these too).  Callers issue their other
// loads, then a scheduling barrier, then use the values: the compiler would otherwise move
// the values to scalar registers, and so wait for them, ahead of the other loads.
__device__ __forceinline__ SeqLen seq_len(const DecodeArgs& a, int bb) {
  const int l = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.len + bb, 4), 0, 0, 0);
  // no append_slot: a zero-sized buffer, whose load reads 0 without touching memory
  const int s = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.append_slot + bb, a.append_slot ? 4 : 0), 0, 0, 0);
  return SeqLen{l, s};
}
__device__ __forceinline__ SeqLen uniform(SeqLen q) {
  return SeqLen{__builtin_amdgcn_readfirstlane(q.len0), __builtin_amdgcn_readfirstlane(q.aslot)};
}

// tokens attended, append slot and this block's slot range (multiples of `align`)
__device__ __forceinline__ Span block_span(const DecodeArgs& a, int c, int align, SeqLen q) {
  Span s;
  if (!a.k_new) { s.n = q.len0; s.app = -1; }
  else if (a.append_slot) { s.n = q.len0; s.app = q.aslot; }
  else { s.n = q.len0 + 1; s.app = q.len0; }
  s.n = min(max(s.n, 0), a.cap);
  if (s.app < 0 || s.app >= a.cap) s.app = -1;
  int per = (s.n + a.n_split - 1) / a.n_split;
  per = (per + align - 1) / align * align;
  s.j0 = c * per;
  s.j1 = min(s.n, s.j0 + per);
  return s;
}

// ------------------------------------------------------------------ new token -> caches
// Each attention block writes its share of dims [c*dpb, (c+1)*dpb) of the new token into slot
// app of the caches (when the token is attended: app < n).  No block reads that slot's
// contents (it is masked), so the write may land at any time during the launch.
template <typename T, int D>
struct NewTok {
  T k, v;
};

template <typename T>
__device__ __forceinline__ T buffer_elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (sizeof(T) == 2) {
    return (T)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  } else {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
}

// NB bytes (4, 8 or 16) at byte offset `off` of a buffer, as raw bits into `out`
template <int NB, typename U>
__device__ __forceinline__ void buffer_bytes(__amdgpu_buffer_rsrc_t r, uint32_t off, U* out) {
  static_assert(NB == 4 || NB == 8 || NB == 16, "bytes");
  if constexpr (NB == 4) {
    const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    __builtin_memcpy(out, &v, 4);
  } else if constexpr (NB == 8) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    __builtin_memcpy(out, &v, 8);
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    __builtin_memcpy(out, &v, 16);
  }
}

// branch-free: lanes without a dim (or calls without a new token) read past a buffer's end
template <typename T, int D>
__device__ __forceinline__ NewTok<T, D> new_token_load(const DecodeArgs& a, int c, size_t pair) {
  const int dpb = (D + a.n_split - 1) / a.n_split, d = c * dpb + (int)threadIdx.x;
  const int bytes = a.k_new ? D * (int)sizeof(T) : 0;
  const uint32_t off = ((int)threadIdx.x < dpb && d < D) ? d * sizeof(T) : D * sizeof(T);
  NewTok<T, D> r;
  r.k = buffer_elem<T>(make_rsrc(reinterpret_cast<const T*>(a.k_new) + pair * D, bytes), off);
  r.v = buffer_elem<T>(make_rsrc(reinterpret_cast<const T*>(a.v_new) + pair * D, bytes), off);
  return r;
}

template <typename T, int D>
__device__ __forceinline__ void new_token_store(const DecodeArgs& a, int c, size_t pair, const Span& sp,
                                                const NewTok<T, D>& r) {
  const int dpb = (D + a.n_split - 1) / a.n_split, d = c * dpb + (int)threadIdx.x;
  if (sp.app >= 0 && sp.app < sp.n && (int)threadIdx.x < dpb && d < D) {
    reinterpret_cast<T*>(a.Kc)[(pair * a.cap + sp.app) * D + d] = r.k;
    reinterpret_cast<T*>(a.Vc)[(pair * D + d) * a.cap + sp.app] = r.v;
  }
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
        const float f = __builtin_amdgcn_exp2f(s_m[w][h] - mx);   // exp2(-inf) = 0
        L = fmaf(s_l[w][h], f, L);
        A = fmaf(s_acc[w][h][dd], f, A);
      }
    }
    // L >= 1 when positive (the max term contributes 2^0), so the hardware reciprocal and
    // log2 are in their accurate range
    pa[i] = L > 0.f ? A * __builtin_amdgcn_rcpf(L) : 0.f;
    if (dd == 0) a.part_lse[(pair * a.n_split + c) * G + h] = L > 0.f ? (mx + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
  }
}

// ------------------------------------------------------------------ read-out rows
// Each attention block computes a slice of the read-out rows num[h][r] = Mat[r] . feat(q_h)
// (feat = phi for the memory, the identity for the moments): thread t takes 8 consecutive
// columns c0 = (t % (D/8)) * 8 of row t / (D/8) of its slice.  The first pass's operands
// (the Mat row piece and q[h][c0 .. c0+8] for every head) are loaded before the K/V stream,
// so their latency overlaps it; rows beyond the first pass (only with very few splits) are
// done after the stream.
template <typename T, int G>
struct ReadoutRegs {
  float4 m0, m1;                    // Mat[row][c0 .. c0+8]
  uint4 qr[G][8 / Vec16<T>::N];     // q[h][c0 .. c0+8], raw
};

// Branch-free: without a read-out (or for lanes without a row) the Mat loads read past a
// buffer's end; q is always there.
template <typename T, int D, int G, int NT>
__device__ __forceinline__ void readout_load(ReadoutRegs<T, G>& r, const DecodeArgs& a, int c, size_t pair,
                                             const T* qp) {
  constexpr int N = Vec16<T>::N, TPR = D / 8;
  const int c0 = (threadIdx.x % TPR) * 8;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < 8 / N; ++j) r.qr[h][j] = *reinterpret_cast<const uint4*>(qp + h * D + c0 + j * N);
  const int rps = (D + a.n_split - 1) / a.n_split;
  const int row = c * rps + threadIdx.x / TPR;
  const bool on = a.mode != KVM_READ_NONE;
  const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.rmat + pair * (size_t)(D * D), on ? D * D * 4 : 0);
  const uint32_t off = (on && (int)threadIdx.x / TPR < rps && row < D) ? (row * D + c0) * 4 : D * D * 4;
  const auto m0 = __builtin_amdgcn_raw_buffer_load_b128(rm, off, 0, 0);
  const auto m1 = __builtin_amdgcn_raw_buffer_load_b128(rm, off + 16, 0, 0);
  r.m0 = make_float4(__uint_as_float(m0[0]), __uint_as_float(m0[1]), __uint_as_float(m0[2]), __uint_as_float(m0[3]));
  r.m1 = make_float4(__uint_as_float(m1[0]), __uint_as_float(m1[1]), __uint_as_float(m1[2]), __uint_as_float(m1[3]));
}

// num[h][row] for one pass of rows, from operands in registers
template <typename T, int D, int G>
__device__ __forceinline__ void readout_pass(const DecodeArgs& a, size_t pair, int rl, int rps, int row,
                                             const float4& m0, const float4& m1, const uint4 (&qr)[G][8 / Vec16<T>::N]) {
  constexpr int N = Vec16<T>::N, TPR = D / 8;
  static_assert(TPR == 8 || TPR == 16, "row split");
  const bool mem = a.mode == KVM_READ_MEMORY;
  const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = 0.f;
#pragma unroll
    for (int j = 0; j < 8 / N; ++j) {
      float f[N];
      Vec16<T>::unpack(qr[h][j], f);
#pragma unroll
      for (int e = 0; e < N; ++e) x = fmaf(mv[j * N + e], mem ? phi_f(f[e]) : f[e], x);
    }
    x = group_sum<TPR>(x);
    if (threadIdx.x % TPR == 0 && rl < rps && row < D) a.num[(pair * G + h) * D + row] = x;
  }
}

template <typename T, int D, int G, int NT>
__device__ __forceinline__ void readout_first(const DecodeArgs& a, int c, size_t pair, const ReadoutRegs<T, G>& r) {
  if (a.mode == KVM_READ_NONE) return;
  constexpr int TPR = D / 8;
  const int rps = (D + a.n_split - 1) / a.n_split;
  const int rl = threadIdx.x / TPR;
  readout_pass<T, D, G>(a, pair, rl, rps, c * rps + rl, r.m0, r.m1, r.qr);
}

template <typename T, int D, int G, int NT>
__device__ __forceinline__ void readout_rest(const DecodeArgs& a, int c, size_t pair, const T* qp) {
  constexpr int N = Vec16<T>::N, TPR = D / 8, RPP = NT / TPR;
  const int rps = (D + a.n_split - 1) / a.n_split;
  if (a.mode == KVM_READ_NONE || rps <= RPP) return;
  const int c0 = (threadIdx.x % TPR) * 8;
  uint4 qr[G][8 / N];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < 8 / N; ++j) qr[h][j] = *reinterpret_cast<const uint4*>(qp + h * D + c0 + j * N);
  for (int pass = 1; pass * RPP < rps; ++pass) {
    const int rl = pass * RPP + threadIdx.x / TPR, row = c * rps + rl;
    float4 m0 = make_float4(0.f, 0.f, 0.f, 0.f), m1 = m0;
    if (rl < rps && row < D) {
      const float* p = a.rmat + pair * (size_t)(D * D) + (size_t)row * D + c0;
      m0 = *reinterpret_cast<const float4*>(p);
      m1 = *reinterpret_cast<const float4*>(p + 4);
    }
    readout_pass<T, D, G>(a, pair, rl, rps, row, m0, m1, qr);
  }
}

// ------------------------------------------------------------------ merge
// grid (D / 32, H_kv, b), 32 * G threads: thread (h, dim) merges the n_split block states of
// one output element in chunk order, then the new token's state, and adds the read-out.
// The 32 threads of a head also form the head's dot products (q . k_new, b . phi(q),
// w_g . q or s_k . q) from D / 32 elements each.  Every load goes out in one round, before
// anything waits: values are kept as raw bits until all loads are issued.
template <typename T, int D, int G, bool PROJ>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  constexpr int E = D / 32;
  const int rb = blockIdx.x, g = blockIdx.y, bb = blockIdx.z;
  const int h = threadIdx.x >> 5, l32 = threadIdx.x & 31, dd = rb * 32 + l32;
  if (h >= G) return;
  args_merge(a);
  const size_t pair = (size_t)bb * a.H_kv + g;
  const SeqLen sl = seq_len(a, bb);
  const float* pl = a.part_lse + pair * a.n_split * G + h;
  const float* pa = a.part_a + pair * a.n_split * (size_t)(G * D) + (size_t)h * D + dd;
  const T* qh = reinterpret_cast<const T*>(a.q) + ((size_t)bb * a.H_q + (size_t)g * G + h) * D + l32 * E;
  const bool mem = a.mode == KVM_READ_MEMORY, mom = a.mode == KVM_READ_MOMENTS;
  // the first 8 block states through buffers sized to n_split: states past it read zeros
  // (lse replaced by -inf below), so these loads sit behind no branch
  float lv[8], av[8];
  {
    const int n8 = min(a.n_split, 8);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.part_lse + pair * a.n_split * G, n8 * G * 4);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.part_a + pair * a.n_split * (size_t)(G * D), n8 * G * D * 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lv[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, (e * G + h) * 4, 0, 0));
      av[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ra, ((e * G + h) * D + dd) * 4, 0, 0));
    }
  }
  // optional inputs through buffers of size 0 when absent (their loads read zeros), so no
  // load sits behind a branch
  constexpr int EB = E * (int)sizeof(T);   // bytes of a head's D / 32 elements
  T qr[E], kr[E], wr[E], qmr[PROJ ? E : 1];
  float xr[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qr[e] = qh[e];
  const int tb = (int)sizeof(T);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(reinterpret_cast<const T*>(a.k_new) + pair * D, a.k_new ? D * tb : 0);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(reinterpret_cast<const T*>(a.v_new) + pair * D, a.k_new ? D * tb : 0);
  // (resource bases are per (sequence, KV head), uniform across the wave; the head goes in
  // the offset)
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(a.num + pair * G * D, (mem || mom) ? G * D * 4 : 0);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc((mem ? a.bvec : a.s_k) + pair * D, (mem || mom) ? D * 4 : 0);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(reinterpret_cast<const T*>(a.w_g) + (size_t)g * G * D, mem ? G * D * tb : 0);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.s_v + pair * D, mom ? D * 4 : 0);
  const __amdgpu_buffer_rsrc_t re = make_rsrc(a.n_e + pair, mom ? 4 : 0);
  buffer_bytes<EB>(rk, l32 * EB, kr);
  if constexpr (PROJ) {   // the projected query addresses the memory
    const __amdgpu_buffer_rsrc_t rqm =
        make_rsrc(reinterpret_cast<const T*>(a.q_mem) + ((size_t)bb * a.H_q + (size_t)g * G) * D, G * D * tb);
    buffer_bytes<EB>(rqm, h * D * tb + l32 * EB, qmr);
  }
  buffer_bytes<EB>(rw, h * D * tb + l32 * EB, wr);
  buffer_bytes<E * 4>(rx, l32 * E * 4, xr);
  const T vr = buffer_elem<T>(rv, dd * tb);
  const float num = buffer_elem<float>(rn, (h * D + dd) * 4);
  const float sv = buffer_elem<float>(rs, dd * 4);
  const int ne = (int)__builtin_amdgcn_raw_buffer_load_b32(re, 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e >= a.n_split) lv[e] = -INFINITY;
  // online merge of the block states in chunk order, 8 at a time
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
  // head dot products: q . k_new, b . phi(q_mem) or s_k . q, w_g . q
  float s_new = 0.f, x0 = 0.f, x1 = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float qv = load_scalar<T>(&qr[e]);
    float qm = qv;
    if constexpr (PROJ) qm = load_scalar<T>(&qmr[e]);
    s_new = fmaf(qv, load_scalar<T>(&kr[e]), s_new);
    x0 = fmaf(xr[e], mem ? phi_f(qm) : qm, x0);
    x1 = fmaf(load_scalar<T>(&wr[e]), qv, x1);
  }
  s_new = group_sum<32>(s_new);
  x0 = group_sum<32>(x0);
  x1 = group_sum<32>(x1);
  // the new token's state: a = v_new, lse = scale q . k_new
  const Span sp = block_span(a, 0, 1, uniform(sl));
  if (sp.app >= 0 && sp.app < sp.n) {
    const float ls = a.scale * s_new;
    const float nm = fmaxf(mx, ls);
    const float f = mx == -INFINITY ? 0.f : __expf(mx - nm);
    const float w = __expf(ls - nm);
    z = fmaf(z, f, w);
    acc = fmaf(acc, f, w * load_scalar<T>(&vr));
    mx = nm;
  }
  float lse = -INFINITY, o = 0.f;
  if (mx != -INFINITY && z > 0.f) {
    lse = mx + __logf(z);
    o = acc / z;
  }
  if (mem) {
    o = fmaf(sigmoid_f(x1), num / (x0 + a.eps), o);
  } else if (mom && ne > 0) {
    const float inv = 1.f / (float)ne;
    const float fE = sv * inv + a.scale * (num - sv * x0 * inv) * inv;
    const float logZ = __logf((float)ne) + a.scale * x0 * inv;
    const float w = sigmoid_f(lse - logZ);
    o = w * o + (1.f - w) * fE;
  }
  a.o[((size_t)bb * a.H_q + g * G + h) * D + dd] = o;
  if (a.lse && dd == 0) a.lse[(size_t)bb * a.H_q + g * G + h] = lse;
}

// ------------------------------------------------------------------ FMA path (any dtype, D)
template <typename T, int D, int G, int NW, bool PROJ>
__global__ __launch_bounds__(NW * 64) void decode_fma_kernel(DecodeArgs a) {
  constexpr int EPL = Vec16<T>::N;   // elements per lane (16 bytes)
  constexpr int LPT = D / EPL;       // lanes per token row
  constexpr int TPI = 64 / LPT;      // token rows per wave instruction
  const int c = blockIdx.x, g = blockIdx.y, bb = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPT, grp = lane / LPT;

  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_acc[NW][G][D];

  const Span sp = block_span(a, c, 1, uniform(seq_len(a, bb)));
  const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)bb * a.H_q + (size_t)g * G) * D;
  const T* qmp = PROJ ? reinterpret_cast<const T*>(a.q_mem) + ((size_t)bb * a.H_q + (size_t)g * G) * D : qp;
  const size_t cache_off = ((size_t)bb * a.H_kv + g) * (size_t)a.cap * D;
  T* Kp = reinterpret_cast<T*>(a.Kc) + cache_off;
  T* Vt = reinterpret_cast<T*>(a.Vc) + cache_off;   // [D][cap]
  const size_t pair = (size_t)bb * a.H_kv + g;
  const NewTok<T, D> nt = new_token_load<T, D>(a, c, pair);
  {
    ReadoutRegs<T, G> rr;
    readout_load<T, D, G, NW * 64>(rr, a, c, pair, qmp);
    readout_first<T, D, G, NW * 64>(a, c, pair, rr);
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
    // the slot that takes the new token is skipped: its cached contents are stale
    const bool skip = (j == sp.app);
    float kf[EPL], vf[EPL];
    Vec16<T>::load(Kp + (size_t)j * D + sub * EPL, kf);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float v = load_scalar<T>(Vt + (size_t)(sub * EPL + e) * a.cap + j);
      vf[e] = skip ? 0.f : v;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s = fmaf(qf[h][e], kf[e], s);
      s = group_sum<LPT>(s);
      const float mn = skip ? m[h] : fmaxf(m[h], s);
      const float cf = skip ? 1.f : exp2f(m[h] - mn);
      const float p = skip ? 0.f : exp2f(s - mn);
      l[h] = fmaf(l[h], cf, p);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(acc[h][e], cf, p * vf[e]);
      m[h] = mn;
    }
  }
  readout_rest<T, D, G, NW * 64>(a, c, pair, qmp);
  new_token_store<T, D>(a, c, pair, sp, nt);
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

// The K rows [cap][D] and V rows [D][cap] of a (sequence, KV head) as buffers; `*_oob` is an
// offset past each buffer's end (loads there read zeros).
struct TileBufs {
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t k_oob, v_oob, v_row;   // v_row: bytes per V row (2 cap)
};

__device__ __forceinline__ uint4 as_uint4(const __attribute__((ext_vector_type(4))) unsigned int& v) {
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// K rows of a tile, permuted: for slot group gq, MFMA row m = 4a + i holds slot a*8 + gq*4 + i.
// With K as the A operand and q as the B operand, S^T = K q^T then leaves the scores of head
// h for slots kg*8 .. kg*8+8 in lane (h, kg) -- the layout in which the P V product takes P
// as its A operand, so P never leaves the registers.
// (slots >= lim read zeros)
__device__ __forceinline__ void tile_load_k(TileRegs& T, int t0, int lim, const TileBufs& B, int m16, int kg) {
#pragma unroll
  for (int gq = 0; gq < 2; ++gq) {
    const int t = t0 + (m16 >> 2) * 8 + gq * 4 + (m16 & 3);
    const uint32_t off = t < lim ? (uint32_t)t * 256u + kg * 16 : B.k_oob;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) T.k[gq][cc] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(B.rk, off + cc * 64, 0, 0));
  }
}

// (8-slot groups starting at or past lim read zeros)
__device__ __forceinline__ void tile_load_v(TileRegs& T, int t0, int lim, const TileBufs& B, int m16, int kg) {
  const int tv = t0 + kg * 8;
  const uint32_t off = tv < lim ? (uint32_t)m16 * B.v_row + (uint32_t)tv * 2u : B.v_oob;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    T.v[dt] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(B.rv, off, dt * 16 * B.v_row, 0));
}

// sc[gq][i] = q[m16] . K[slot kg*8 + gq*4 + i]
__device__ __forceinline__ void tile_scores(const TileRegs& T, const bf16x8_t (&qb)[4], f32x4_t (&sc)[2]) {
#pragma unroll
  for (int gq = 0; gq < 2; ++gq) {
    sc[gq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      bf16x8_t ka;
      __builtin_memcpy(&ka, &T.k[gq][cc], 16);
      sc[gq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[cc], sc[gq], 0, 0, 0);
    }
  }
}

// bf16 hi + lo split of 8 probabilities (16-bit accurate P)
__device__ __forceinline__ void split_bf16(const float (&p)[8], bf16x8_t& hi, bf16x8_t& lo) {
  float r[8];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const bf16x2_t h = __builtin_convertvector(f32x2_t{p[j], p[j + 1]}, bf16x2_t);
    hi[j] = h[0];
    hi[j + 1] = h[1];
    r[j] = p[j] - (float)h[0];
    r[j + 1] = p[j + 1] - (float)h[1];
  }
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const bf16x2_t l2 = __builtin_convertvector(f32x2_t{r[j], r[j + 1]}, bf16x2_t);
    lo[j] = l2[0];
    lo[j + 1] = l2[1];
  }
}

// Online softmax of one tile and acc = acc * cf + P V.  Lane (h = m16, kg) holds head h's
// scores for slots kg*8 .. +8; m is head h's running max (equal in its four lanes), l this
// lane's share of the running sum.  Slots >= lim (the length) and the new token's slot app
// are masked; tiles with neither skip the masking.
template <int G>
__device__ __forceinline__ void tile_pv(TileRegs& T, const f32x4_t (&sc)[2], int t0, int lim, int app, float qs,
                                        int m16, int kg, float& m, float& l, f32x4_t (&acc)[8]) {
  const int s0 = t0 + kg * 8;
  const bool full = t0 + 32 <= lim && (unsigned)(app - t0) >= 32u;   // wave-uniform
  float x[8];
#pragma unroll
  for (int gq = 0; gq < 2; ++gq)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[gq * 4 + i] = sc[gq][i] * qs;
  const int valid = lim - s0;   // slots of this lane's group below the length
  const int ap = app - s0;      // position of the new token's slot in the group
  if (!full) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j >= valid || j == ap) x[j] = -INFINITY;
    // V fix-ups (P is 0 there, but the bytes may be stale or not finite): zero the slots
    // at or past the length and the new token's slot.
    if (valid < 8 || (ap >= 0 && ap < 8)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint32_t w[4] = {T.v[dt].x, T.v[dt].y, T.v[dt].z, T.v[dt].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t keep = (e >= valid || e == ap) ? 0u : 0xffffu;
          w[e >> 1] &= (e & 1) ? ((keep << 16) | 0xffffu) : (keep | 0xffff0000u);
        }
        T.v[dt] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
  float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  mx = fmaxf(mx, swz_xor16(mx));
  mx = fmaxf(mx, shfl_xor32(mx));
  const float mn = fmaxf(m, mx);
  const float msafe = mn == -INFINITY ? 0.f : mn;
  const float cf = __builtin_amdgcn_exp2f(m - msafe);
  float p[8], ps = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = __builtin_amdgcn_exp2f(x[j] - msafe);
    ps += p[j];
  }
  l = fmaf(l, cf, ps);
  m = mn;
  bf16x8_t pha, pla;
  split_bf16(p, pha, pla);
  // acc rows are heads 4*kg + i: their rescale factors come from lanes 4*kg + i
  float cr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float c0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cf), i));
    if (G > 4) {
      const float c1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cf), 4 + i));
      cr[i] = kg == 1 ? c1 : c0;
    } else {
      cr[i] = c0;
    }
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[dt][i] *= cr[i];
    bf16x8_t vb;
    __builtin_memcpy(&vb, &T.v[dt], 16);
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pha, vb, acc[dt], 0, 0, 0);
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pla, vb, acc[dt], 0, 0, 0);
  }
}

// ------------------------------------------------------------------ matrix-core path
// bf16, D = 128.  Tiles of 32 slots, one per wave in flight.  The slots are dealt to the
// n_split blocks of a (sequence, KV head) in chunks of 128 (a tile per wave), round robin:
// block c takes chunks c, c + n_split, ...  So a block's first chunk does not depend on the
// sequence length, and its loads go out before the length has arrived (it is bounded by
// cap; slots at or past the length are masked once it is known); the blocks' shares differ
// by at most one chunk for any length; and 128-slot chunks keep every 128-byte line of a V
// row (cap a multiple of 64) within one block.
constexpr int WPE = 2;   // waves per SIMD: two 4-wave blocks per compute unit
template <int G, bool PROJ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int D = 128, NW = 4, TILE = 32, STEP = NW * TILE;
  static_assert(G <= 8, "G");
  const int c = blockIdx.x, g = blockIdx.y, bb = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: tile starts live in SGPRs
  const int m16 = lane & 15, kg = lane >> 4;

  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_acc[NW][G][D];

  args_early(a);
  const size_t pair = (size_t)bb * a.H_kv + g;
  // q and the read-out operands do not depend on the sequence length: their loads go out
  // while the length is still being read
  const SeqLen sl = seq_len(a, bb);
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)bb * a.H_q + (size_t)g * G) * D;
  const uint16_t* qmp =
      PROJ ? reinterpret_cast<const uint16_t*>(a.q_mem) + ((size_t)bb * a.H_q + (size_t)g * G) * D : qp;
  ReadoutRegs<uint16_t, G> rr;
  readout_load<uint16_t, D, G, NW * 64>(rr, a, c, pair, qmp);
  const NewTok<uint16_t, D> nt = new_token_load<uint16_t, D>(a, c, pair);

  // B operand of S^T = K q^T: lane (head m16, k group kg) holds q[m16][cc*32 + kg*8 .. +8]
  // (heads >= G read past the buffer: zeros)
  bf16x8_t qb[4];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qp, G * D * 2);
    const uint32_t off = m16 < G ? (uint32_t)m16 * D * 2 + kg * 16 : G * D * 2;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const uint4 v = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rq, off + cc * 64, 0, 0));
      __builtin_memcpy(&qb[cc], &v, 16);
    }
  }
  TileBufs B;
  B.rk = make_rsrc(reinterpret_cast<const uint16_t*>(a.Kc) + pair * (size_t)a.cap * D, a.cap * D * 2);
  B.rv = make_rsrc(reinterpret_cast<const uint16_t*>(a.Vc) + pair * (size_t)a.cap * D, a.cap * D * 2);
  B.k_oob = (uint32_t)a.cap * D * 2;
  B.v_oob = (uint32_t)a.cap * D * 2;
  B.v_row = (uint32_t)a.cap * 2;
  // the first tile, bounded by cap
  TileRegs ta;
  int t0 = c * STEP + wave * TILE;
  tile_load_k(ta, t0, a.cap, B, m16, kg);
  tile_load_v(ta, t0, a.cap, B, m16, kg);
  __builtin_amdgcn_sched_barrier(0);
  const Span sp = block_span(a, 0, 1, uniform(sl));   // n, app (j0, j1 unused)

  // One tile in flight per wave: once a tile's scores are done its registers take the next
  // tile's K loads (bounded by the length n), once P V is done its V loads.  (Two tiles in
  // flight per wave measured slower: with every load of the launch issued at once, each
  // wave's data arrives late.)  Loads past the bound read zeros, so the loop's loads are
  // unconditional.
  readout_first<uint16_t, D, G, NW * 64>(a, c, pair, rr);
  const int stride = a.n_split * STEP;

  const float qs = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f;
  f32x4_t acc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (; t0 < sp.n; t0 += stride) {
    f32x4_t sc[2];
    tile_scores(ta, qb, sc);
    tile_load_k(ta, t0 + stride, sp.n, B, m16, kg);
    tile_pv<G>(ta, sc, t0, sp.n, sp.app, qs, m16, kg, m, l, acc);
    tile_load_v(ta, t0 + stride, sp.n, B, m16, kg);
  }
  readout_rest<uint16_t, D, G, NW * 64>(a, c, pair, qmp);
  new_token_store<uint16_t, D>(a, c, pair, sp, nt);
  // wave state -> LDS: head h's max and sum (over its four lanes) from lane h, acc rows
  // 4*kg + i from the lanes of group kg
  l += swz_xor16(l);
  l += shfl_xor32(l);
  if (kg == 0 && m16 < G) { s_m[wave][m16] = m; s_l[wave][m16] = l; }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * kg + i;
    if (h < G) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) s_acc[wave][h][dt * 16 + m16] = acc[dt][i];
    }
  }
  __syncthreads();
  write_partial<D, G, NW>(a, c, g, bb, s_m, s_l, s_acc);
}

__global__ void len_add_kernel(int32_t* len, int b, int delta) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < b) len[i] += delta;
}

// Splits per (sequence, KV head): the most that keep the grid within one round of two
// attention blocks per compute unit (256 on this part).  A grid that overfills the round
// leaves a second, partial round; one that does not divide evenly leaves some units with
// twice the work of others -- both measured 15-30% slower than a full, even round.
// Without a read-out each block should hold at least one 128-slot chunk.  With one, up to 8
// splits even for short caches: the blocks also share the D read-out rows of M (or S), and
// one block reading a whole 64 KB matrix in passes of 16 rows is the longest chain of a
// short cache's step (measured, MomentKV batch 4, 36 layers: B = 128 13.4 -> 8.9 us per
// layer-step, B = 256 12.3 -> 9.3 us; 16 splits were slower than 8).
static int auto_split(const kvm_decode_desc* d) {
  if (d->n_split > 0) return d->n_split;
  constexpr int kBlockSlots = 2 * 256;
  const int pairs = d->b * d->H_kv;
  int s = std::max(1, kBlockSlots / pairs);
  s = std::min(s, std::max(d->mode != KVM_READ_NONE ? 8 : 1, d->cap / 128));
  return std::min(s, 64);
}

struct DecodeWs {
  size_t a, lse, num, total;
};
static DecodeWs decode_ws(const kvm_decode_desc* d, int ns) {
  const int G = d->H_q / d->H_kv;
  const size_t pairs = (size_t)d->b * d->H_kv;
  DecodeWs w;
  w.a = 0;
  w.lse = align_up(w.a + pairs * ns * G * d->d * sizeof(float), 256);
  w.num = align_up(w.lse + pairs * ns * G * sizeof(float), 256);
  w.total = align_up(w.num + pairs * G * d->d * sizeof(float), 256);
  return w;
}

template <typename T, int D, int G, bool PROJ>
static void launch_decode_p(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.n_split, a.H_kv, a.b);
  if constexpr (std::is_same<T, uint16_t>::value && D == 128)
    hipLaunchKernelGGL((decode_mfma_kernel<G, PROJ>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((decode_fma_kernel<T, D, G, 4, PROJ>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL((decode_merge_kernel<T, D, G, PROJ>), dim3(D / 32, a.H_kv, a.b), dim3(32 * G), 0, st, a);
}

// the read-out's projected query is a compile-time switch, so the plain path is unchanged
template <typename T, int D, int G>
static void launch_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.q_mem != a.q) launch_decode_p<T, D, G, true>(a, st);
  else launch_decode_p<T, D, G, false>(a, st);
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

// Validation and launch shared by both decode entry points; ws == nullptr asks for the
// library's own scratch array instead of a caller workspace.
static kvm_status decode_entry(const kvm_decode_desc* d, const void* q, const void* k_new, const void* v_new,
                               const int32_t* append_slot, void* Kc, void* Vc, const int32_t* len, const float* M,
                               const float* bvec, const void* w_g, const void* q_mem, const int32_t* n_e,
                               const float* s_k, const float* s_v, const float* S, float* o, float* lse, void* ws,
                               size_t ws_bytes, bool own_scratch, void* stream);

extern "C" kvm_status kvm_decode_attn_mem(const kvm_decode_desc* d, const void* q, const void* k_new,
                                          const void* v_new, const int32_t* append_slot, void* Kc,
                                          void* Vc, const int32_t* len, const float* M,
                                          const float* bvec, const void* w_g, const void* q_mem,
                                          const int32_t* n_e, const float* s_k, const float* s_v,
                                          const float* S, float* o, float* lse, void* ws,
                                          size_t ws_bytes, void* stream) {
  return decode_entry(d, q, k_new, v_new, append_slot, Kc, Vc, len, M, bvec, w_g, q_mem, n_e, s_k, s_v, S, o, lse,
                      ws, ws_bytes, false, stream);
}

// ------------------------------------------------------------------ no-allocation variant
// The split states of kvm_decode_attn_mem_noalloc live in one file-scope device array per GPU
// (the runtime gives each device its own copy).  Host code never passes the array's name to a
// kernel: that name is a host-side stand-in, not a device address.  The device address comes
// from hipGetSymbolAddress, once per device, on the first call with that device current.
// The decode writes every scratch word it reads within the same call, so nothing in the
// array needs clearing between calls; calls that overlap on one GPU race on it.
static constexpr size_t kDecodeScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char decode_scratch[kDecodeScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

static kvm_status decode_scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return check_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return set_error(KVM_ERR_ARCH, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(decode_scratch));
    if (e != hipSuccess || p == nullptr) return check_hip(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                          "hipGetSymbolAddress(decode scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVM_OK;
}

extern "C" size_t kvm_decode_noalloc_max_bytes(void) { return kDecodeScratchBytes; }

extern "C" kvm_status kvm_decode_attn_mem_noalloc(const kvm_decode_desc* d, const void* q, const void* k_new,
                                                  const void* v_new, const int32_t* append_slot, void* Kc,
                                                  void* Vc, const int32_t* len, const float* M,
                                                  const float* bvec, const void* w_g, const void* q_mem,
                                                  const int32_t* n_e, const float* s_k, const float* s_v,
                                                  const float* S, float* o, float* lse, void* stream) {
  return decode_entry(d, q, k_new, v_new, append_slot, Kc, Vc, len, M, bvec, w_g, q_mem, n_e, s_k, s_v, S, o, lse,
                      nullptr, 0, true, stream);
}

static kvm_status decode_entry(const kvm_decode_desc* d, const void* q, const void* k_new, const void* v_new,
                               const int32_t* append_slot, void* Kc, void* Vc, const int32_t* len, const float* M,
                               const float* bvec, const void* w_g, const void* q_mem, const int32_t* n_e,
                               const float* s_k, const float* s_v, const float* S, float* o, float* lse, void* ws,
                               size_t ws_bytes, bool own_scratch, void* stream) {
  KVM_PTR(d);
  KVM_REQUIRE(d->b > 0 && d->H_q > 0 && d->H_kv > 0 && d->cap > 0, KVM_ERR_SHAPE,
              "b, H_q, H_kv and cap must be positive");
  KVM_REQUIRE(d->cap % 8 == 0, KVM_ERR_SHAPE, "cap %d is not a multiple of 8", d->cap);
  KVM_REQUIRE((int64_t)d->cap * 256 <= INT32_MAX, KVM_ERR_SHAPE, "cap %d above 8388607 slots", d->cap);
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
  KVM_REQUIRE(q_mem == nullptr || d->mode == KVM_READ_MEMORY, KVM_ERR_RANGE,
              "q_mem is read only by the memory read-out (mode %d)", d->mode);
  KVM_OPT_ALIGNED(q_mem);
  if (d->mode == KVM_READ_MOMENTS) {
    KVM_PTR_ALIGNED(n_e); KVM_PTR_ALIGNED(s_k); KVM_PTR_ALIGNED(s_v); KVM_PTR_ALIGNED(S);
  }
  const int ns = auto_split(d);
  const DecodeWs w = decode_ws(d, ns);
  if (own_scratch) {
    KVM_REQUIRE(w.total <= kDecodeScratchBytes, KVM_ERR_WORKSPACE,
                "kvm_decode_attn_mem_noalloc: this shape needs %zu bytes of split states, above the %zu-byte "
                "scratch array (use kvm_decode_attn_mem with a workspace, or fewer splits)",
                w.total, kDecodeScratchBytes);
  } else {
    KVM_REQUIRE(ws != nullptr && ws_bytes >= w.total, KVM_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
    KVM_ALIGNED(ws);
  }
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;
  if (own_scratch) {
    st = decode_scratch_ptr(&ws);
    if (st != KVM_OK) return st;
  }

  DecodeArgs a{};
  a.q = q; a.q_mem = q_mem ? q_mem : q; a.k_new = k_new; a.v_new = v_new; a.append_slot = append_slot;
  a.Kc = Kc; a.Vc = Vc; a.len = len; a.M = M; a.bvec = bvec; a.w_g = w_g;
  a.n_e = n_e; a.s_k = s_k; a.s_v = s_v; a.S = S; a.o = o; a.lse = lse;
  a.rmat = d->mode == KVM_READ_MEMORY ? M : S;
  char* base = static_cast<char*>(ws);
  a.part_a = reinterpret_cast<float*>(base + w.a);
  a.part_lse = reinterpret_cast<float*>(base + w.lse);
  a.num = reinterpret_cast<float*>(base + w.num);
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

// q_mem[r] = W_m q[r] for rows r of [rows, D]: 4 rows per block, thread i forms output dim i
// from W_m's row i (fp32 accumulation, stored in the query's dtype).
template <typename T, int D>
__global__ __launch_bounds__(D) void mem_query_kernel(const T* q, const T* W, T* out, int rows) {
  constexpr int N = Vec16<T>::N, RPB = 4;
  const int r0 = blockIdx.x * RPB, i = threadIdx.x;
  __shared__ float sq[RPB][D];
#pragma unroll
  for (int u = 0; u < RPB; ++u)
    sq[u][i] = r0 + u < rows ? load_scalar<T>(q + (size_t)(r0 + u) * D + i) : 0.f;
  float w[D];
#pragma unroll
  for (int c = 0; c < D; c += N) {
    float t[N];
    Vec16<T>::load(W + (size_t)i * D + c, t);
#pragma unroll
    for (int e = 0; e < N; ++e) w[c + e] = t[e];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < RPB; ++u) {
    float x = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) x = fmaf(w[c], sq[u][c], x);
    if (r0 + u < rows) {
      if constexpr (sizeof(T) == 2) {
        const __bf16 h = (__bf16)x;
        __builtin_memcpy(out + (size_t)(r0 + u) * D + i, &h, 2);
      } else {
        out[(size_t)(r0 + u) * D + i] = x;
      }
    }
  }
}

extern "C" kvm_status kvm_mem_query(int32_t rows, int32_t d, int32_t dtype, const void* q, const void* W_m,
                                    void* q_mem, void* stream) {
  KVM_REQUIRE(rows > 0, KVM_ERR_SHAPE, "rows must be positive");
  KVM_REQUIRE(d == 64 || d == 128, KVM_ERR_SHAPE, "head dim %d not in {64, 128}", d);
  KVM_REQUIRE(dtype == KVM_F32 || dtype == KVM_BF16, KVM_ERR_DTYPE, "dtype %d", dtype);
  KVM_PTR_ALIGNED(q); KVM_PTR_ALIGNED(W_m); KVM_PTR_ALIGNED(q_mem);
  KVM_REQUIRE(q_mem != q, KVM_ERR_RANGE, "q_mem must not alias q");
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;
  const dim3 grid((rows + 3) / 4);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == KVM_BF16) {
    const auto* qb = static_cast<const uint16_t*>(q);
    const auto* wb = static_cast<const uint16_t*>(W_m);
    auto* ob = static_cast<uint16_t*>(q_mem);
    if (d == 128) hipLaunchKernelGGL((mem_query_kernel<uint16_t, 128>), grid, dim3(128), 0, s, qb, wb, ob, rows);
    else hipLaunchKernelGGL((mem_query_kernel<uint16_t, 64>), grid, dim3(64), 0, s, qb, wb, ob, rows);
  } else {
    const auto* qf = static_cast<const float*>(q);
    const auto* wf = static_cast<const float*>(W_m);
    auto* of = static_cast<float*>(q_mem);
    if (d == 128) hipLaunchKernelGGL((mem_query_kernel<float, 128>), grid, dim3(128), 0, s, qf, wf, of, rows);
    else hipLaunchKernelGGL((mem_query_kernel<float, 64>), grid, dim3(64), 0, s, qf, wf, of, rows);
  }
  return check_hip(hipGetLastError(), "mem_query launch");
}

extern "C" kvm_status kvm_len_add(int32_t* len, int32_t b, int32_t delta, void* stream) {
  KVM_PTR_ALIGNED(len);
  KVM_REQUIRE(b > 0, KVM_ERR_SHAPE, "b must be positive");
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;
  hipLaunchKernelGGL(len_add_kernel, dim3((b + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), len, b, delta);
  return check_hip(hipGetLastError(), "len_add launch");
}
