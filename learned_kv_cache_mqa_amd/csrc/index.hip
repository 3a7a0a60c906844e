// A1-A3: the learned MQA-style indexer and its per-key importance [IM 2.A].
//
//   k_hat[t]   = RMSNorm(W_kI x_t)                       one shared key per token
//   q~[s,h]    = sigmoid(W_g[h].x_s) RMSNorm(W_qI[h] q_{s,c(h)}) / sqrt(d_I)
//   I[t]       = max_{s: pos(s) >= t} sum_h relu(q~[s,h] . k_hat[t])
// The gate is folded into the query (g > 0, so g relu(x) = relu(g x)).
//
// Kernels:
//  keyproj_mfma  bf16 X, d_I = 64: v_mfma_f32_32x32x16_bf16, one wave per 32 tokens, the
//                W_kI chunk of each 64-wide k step staged once per block in LDS; X rows
//                stream from HBM straight into MFMA operand registers (64 contiguous bytes
//                per lane).  RMSNorm in the epilogue with 32-lane DPP reductions.
//  query         per (sequence, window query): gate dots and the per-head down-projection
//                (16 lanes per output row), RMSNorm per head.
//  score_mfma    H_I = 32, d_I = 64: a 32 x 32 tile is (32 heads of one query) x (32 keys),
//                so the head sum is an in-lane sum plus one cross-half add.  Operands are
//                split fp16 hi + lo (lo scaled by 2^11): q.k = hi.hi + 2^-11 (hi.lo' + lo'.hi)
//                on v_mfma_f32_32x32x16_f16, ~22 bits per operand, so I keeps near-fp32
//                accuracy.  Each wave keeps its 64 keys' operands in registers and streams
//                the window queries through LDS (4 per block barrier); the running max
//                stays in registers.  The MFMAs of one key tile run beside the VALU
//                epilogue of the other.  The three products per q.k bound it: without
//                the epilogue the kernel takes ~80% of its time, on the matrix cores.
//  keyproj_valu / score_valu: fp32 FMA versions for the other shapes.
#include "common.hpp"

namespace kvm {

struct IndexArgs {
  const void* X;
  const void* Qwin;
  const void* W_kI;
  const float* gamma_k;
  const void* W_qI;
  const float* gamma_q;
  const void* W_g;
  float* I;
  float* khat;   // [b, L, d_I]
  float* qt;     // [b, W, H_I, d_I]
  size_t kh_stride;   // elements between sequences in the key projection's khat writes (L d_I)
  float* gate;   // [b, W, H_I] head gates from the key kernel (matrix-core path), or null
  int b, L, D, H_q, d, H_I, d_I, W;
  float eps;
};

// ------------------------------------------------------------------ A1: keys, matrix cores
constexpr int kKpPitch = 36;  // words per LDS row of a weight chunk (64 bf16 + 8 pad)

// Blocks that launch at most this many leave CUs idle (256 CUs): such grids take launch
// shapes with smaller blocks.
constexpr int kFillBlocks = 256;

// Key projection epilogue: lane holds output column m (tile 0) and 32 + m (tile 1) for 16
// token rows; RMS-normalise each row, scale by gamma_k, store into kout (the sequence's
// rows); window rows (the last W of L) also store their head gates sigmoid(W_g x) into
// gout (the sequence's [W, H_I]).  Plain values only: with the argument struct passed by
// reference the compiler keeps a private copy and spills the streaming variant.
__device__ __forceinline__ void keyproj_epilogue(f32x16_t acc0, f32x16_t acc1, f32x16_t acc2, const float* gamma_k,
                                                 float* kout, float* gout, int L, int W, int H_I, float eps,
                                                 bool gate, int t0, int m, int kg) {
  const float g0 = gamma_k[m], g1 = gamma_k[32 + m];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = 8 * (j / 4) + 4 * kg + (j % 4);
    float ss = acc0[j] * acc0[j] + acc1[j] * acc1[j];
    ss = group_sum<32>(ss);
    const float r = rsqrtf(ss * (1.f / 64.f) + eps);
    const int t = t0 + row;
    if (t < L) {
      kout[(size_t)t * 64 + m] = g0 * acc0[j] * r;
      kout[(size_t)t * 64 + 32 + m] = g1 * acc1[j] * r;
      if (gate && t >= L - W && m < H_I) gout[(size_t)(t - (L - W)) * H_I + m] = sigmoid_f(acc2[j]);
    }
  }
}


// Block: 128 tokens (4 waves x 32); outputs = d_I = 64 key dims (2 tiles of 32) plus, in
// blocks that hold window positions, a third tile with the H_I (<= 32) gate logits
// W_g[h] . x, so X is read once for both.  X streams through a ring of XS k-steps in
// registers; the weight chunk of each k-step is staged in LDS (double-buffered).
// Key projection launch shape: 16 waves x 32 tokens per block share each staged weight
// chunk, so the weights' L2 traffic per token is a sixteenth of the X stream's; 4 waves per
// SIMD with two k-steps of X in flight per wave.
constexpr int kKpWPE = 4;                   // waves per SIMD
constexpr int kKpXS = 2;                    // k-steps of X in flight per wave
constexpr int kKpNW = 16;                   // waves per block, 32 tokens each
constexpr int kKpTB = kKpNW * 32;           // tokens per block
__global__ __launch_bounds__(kKpNW * 64) __attribute__((amdgpu_waves_per_eu(kKpWPE, kKpWPE))) void keyproj_mfma_kernel(IndexArgs a) {
  constexpr int XS = kKpXS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bb = blockIdx.y;
  const int tb0 = blockIdx.x * kKpTB, t0 = tb0 + wave * 32;
  const int m = lane & 31, kg = lane >> 5;
  const bool gate = tb0 + kKpTB - 1 >= a.L - a.W && a.gate != nullptr;   // block-uniform
  __shared__ uint32_t sW[2][96 * kKpPitch];
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.X) + (size_t)bb * a.L * a.D;
  const uint16_t* Wk = reinterpret_cast<const uint16_t*>(a.W_kI);
  const uint16_t* Wg = reinterpret_cast<const uint16_t*>(a.W_g);
  const int tok = min(t0 + m, a.L - 1);        // clamp: rows past L compute garbage, never stored
  const uint16_t* xrow = X + (size_t)tok * a.D + kg * 8;   // MFMA j of a k-step: dims j*16 + kg*8 .. +8

  f32x16_t acc0, acc1, acc2;
#pragma unroll
  for (int j = 0; j < 16; ++j) { acc0[j] = 0.f; acc1[j] = 0.f; acc2[j] = 0.f; }

  // weight chunk rows: 0..63 W_kI, 64..95 W_g (zero beyond H_I); 768 uint4 over the threads
  constexpr int NT = kKpNW * 64, NE = (768 + NT - 1) / NT;
  const int wq = tid & 7;
  const int wrows = gate ? 96 : 64;   // rows in use
  auto wsrc = [&](int i, int k0) -> uint4 {
    const int row = (tid + i * NT) >> 3;
    if (row < 64) return *reinterpret_cast<const uint4*>(Wk + (size_t)row * a.D + k0 + wq * 8);
    if (row < wrows && row - 64 < a.H_I) return *reinterpret_cast<const uint4*>(Wg + (size_t)(row - 64) * a.D + k0 + wq * 8);
    return make_uint4(0, 0, 0, 0);
  };
  const int nk = a.D / 64;
  // Each block starts its k loop at a different k-step so that the blocks' concurrent X
  // reads (rows 2*D bytes apart) spread over the HBM channels instead of all hitting the
  // same column offset at once.
  const int rot = (int)((blockIdx.x * 7u + blockIdx.y * 13u) % (unsigned)nk);
  auto kofs = [&](int ks) { int k = ks + rot; return (k >= nk ? k - nk : k) * 64; };
  // Weight chunks run two k-steps ahead: the chunk of step ks + 2 is loaded at step ks into
  // one register set while the other set (step ks + 1) is written to the idle LDS buffer.
  uint4 w[2][NE];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < NE; ++i) w[h][i] = make_uint4(0, 0, 0, 0);
  auto wload = [&](int h, int ks) {
    const int k = kofs(ks);
#pragma unroll
    for (int i = 0; i < NE; ++i)
      if (((tid + i * NT) >> 3) < wrows) w[h][i] = wsrc(i, k);
  };
  auto wstore = [&](int h, int buf) {
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int e = tid + i * NT;
      if ((e >> 3) < wrows) *reinterpret_cast<uint4*>(&sW[buf][(e >> 3) * kKpPitch + wq * 4]) = w[h][i];
    }
  };
  wload(0, 0);
  if (nk > 1) wload(1, 1);
  wstore(0, 0);

  uint4 xr[XS][4];
#pragma unroll
  for (int st = 0; st < XS; ++st)
    if (st < nk)
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[st][i] = *reinterpret_cast<const uint4*>(xrow + kofs(st) + i * 16);
  __syncthreads();
  static_assert(XS % 2 == 0, "register set of a step follows from st");
  for (int k0 = 0; k0 < nk; k0 += XS) {
#pragma unroll
    for (int st = 0; st < XS; ++st) {
      const int ks = k0 + st;
      if (ks >= nk) break;
      const int buf = st & 1;   // == ks & 1
      if (ks + 2 < nk) wload(st & 1, ks + 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8_t A, B0, B1, B2;
        __builtin_memcpy(&A, &xr[st][j], 16);
        const uint4 b0 = *reinterpret_cast<const uint4*>(&sW[buf][m * kKpPitch + j * 8 + kg * 4]);
        const uint4 b1 = *reinterpret_cast<const uint4*>(&sW[buf][(32 + m) * kKpPitch + j * 8 + kg * 4]);
        __builtin_memcpy(&B0, &b0, 16);
        __builtin_memcpy(&B1, &b1, 16);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B1, acc1, 0, 0, 0);
        if (gate) {
          const uint4 b2 = *reinterpret_cast<const uint4*>(&sW[buf][(64 + m) * kKpPitch + j * 8 + kg * 4]);
          __builtin_memcpy(&B2, &b2, 16);
          acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B2, acc2, 0, 0, 0);
        }
      }
      if (ks + XS < nk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xr[st][i] = *reinterpret_cast<const uint4*>(xrow + kofs(ks + XS) + i * 16);
      }
      if (ks + 1 < nk) wstore((st + 1) & 1, buf ^ 1);
      __syncthreads();
    }
  }
  keyproj_epilogue(acc0, acc1, acc2, a.gamma_k, a.khat + (size_t)bb * a.kh_stride,
                   gate ? a.gate + (size_t)bb * a.W * a.H_I : nullptr, a.L, a.W, a.H_I, a.eps, gate, t0, m, kg);
}

// Key projection for grids that would leave CUs idle (short prefill chunks, small batches):
// the same contraction as keyproj_mfma_kernel in blocks of NW compute waves x 32 tokens plus
// one producer wave, so a chunk of 4096 tokens x batch 8 still gives every CU a block (NW = 4;
// NW = 2 where even that grid is short, e.g. batch 1: 74 instead of 82 us at 16K tokens).
//  - Fewer waves per CU must each keep more of X in flight: XS k-steps per wave, all loads
//    unconditional through a buffer resource (rows past L and steps past the last read as
//    zeros without touching memory), so the wait before each step counts only X loads.
//  - A wave's loads complete in issue order, so the weight chunks are moved by the producer
//    alone: a compute wave that also loaded weights would wait at every step for the X
//    loads issued before them.  The producer keeps WD chunks in flight (a step here is short
//    and the weights come from an L2 that the X stream keeps busy) and writes each into the
//    idle half of the LDS double buffer one step ahead of its use.
// Barriers: every wave, producer or not, passes one after the prologue and one per k-step.
constexpr int kKpsNW = 4;   // compute waves per block
constexpr int kKpsXS = 8;   // k-steps of X in flight per compute wave
constexpr int kKpsWD = 4;   // weight chunks in flight in the producer
template <int NW, int XS, int WD>
__global__ __launch_bounds__((NW + 1) * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void keyproj_stream_kernel(IndexArgs a) {
  constexpr int TB = NW * 32;   // tokens per block
  // the wave index through readfirstlane: the producer branch and the X buffer resource stay
  // scalar (a per-lane value there turns every load into a loop over the distinct lane values)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave == NW;   // wave-uniform
  const int bb = blockIdx.y;
  const int tb0 = blockIdx.x * TB, t0 = tb0 + (producer ? 0 : wave) * 32;
  const int m = lane & 31, kg = lane >> 5;
  const bool gate = tb0 + TB - 1 >= a.L - a.W && a.gate != nullptr;   // block-uniform
  __shared__ uint32_t sW[2][96 * kKpPitch];
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.X) + (size_t)bb * a.L * a.D;
  const int nk = a.D / 64;
  // Each block starts its k loop at a different k-step (spreads the blocks' concurrent X
  // reads over the HBM channels).
  const int rot = (int)((blockIdx.x * 7u + blockIdx.y * 13u) % (unsigned)nk);
  auto kofs = [&](int ks) { int k = ks + rot; return (k >= nk ? k - nk : k) * 64; };

  if (producer) {
    // weight chunk rows: 0..63 W_kI, 64..95 W_g (zeros past H_I, and outside the window's
    // blocks); lane moves 16 bytes of rows 8 i + (lane >> 3), i = 0..11 (i < 8: W_kI)
    const __amdgpu_buffer_rsrc_t rWk = make_rsrc(a.W_kI, 64 * a.D * 2);
    const __amdgpu_buffer_rsrc_t rWg = make_rsrc(a.W_g, (gate ? a.H_I : 0) * a.D * 2);
    const int wq = lane & 7, wr = lane >> 3;
    const int nrow = gate ? 12 : 8;   // row groups of 8 in use
    uint4 w[WD][12];
    // chunk j lives in register set j % WD; chunks past the last step read zeros (no branch,
    // so the wait before each store counts only the chunks issued before it)
    auto wload = [&](int h, int ks) {
      const bool v = ks < nk;
      const int col = (kofs(v ? ks : 0) + wq * 8) * 2;
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        const int off = (8 * (i & 7) + wr) * a.D * 2 + col;
        w[h][i] = load16(i < 8 ? rWk : rWg, v ? off : 0x40000000);
      }
    };
    auto wstore = [&](int h, int buf) {
#pragma unroll
      for (int i = 0; i < 12; ++i)
        if (i < nrow) *reinterpret_cast<uint4*>(&sW[buf][(8 * i + wr) * kKpPitch + wq * 4]) = w[h][i];
    };
#pragma unroll
    for (int h = 0; h < WD; ++h) wload(h, h);
    wstore(0, 0);
    wload(0, WD);   // set 0 is free again: chunk WD (step ks stores chunk ks + 1, loads ks + 1 + WD)
    __syncthreads();
    static_assert(WD % 2 == 0, "LDS buffer and register set of a step follow from the unrolled index");
    for (int k0 = 0; k0 < nk; k0 += WD) {
#pragma unroll
      for (int u = 0; u < WD; ++u) {
        const int ks = k0 + u;
        if (ks >= nk) break;
        const int hs = (u + 1) % WD;   // set of chunk ks + 1
        if (ks + 1 < nk) wstore(hs, (u + 1) & 1);
        wload(hs, ks + 1 + WD);
        __syncthreads();
      }
    }
    return;
  }

  // The wave's 32 X rows; MFMA j of a k-step takes dims j*16 + kg*8 .. +8 of row m.
  const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(32, a.L - t0)));
  const int xrow0 = __builtin_amdgcn_readfirstlane(min(t0, a.L - 1));
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(X + (size_t)xrow0 * a.D, nrows * a.D * 2);
  const int xoff0 = (m * a.D + kg * 8) * 2;
  auto xoff = [&](int ks) { return ks < nk ? xoff0 + kofs(ks) * 2 : 0x40000000; };
  f32x16_t acc0, acc1, acc2;
#pragma unroll
  for (int j = 0; j < 16; ++j) { acc0[j] = 0.f; acc1[j] = 0.f; acc2[j] = 0.f; }
  uint4 xr[XS][4];
#pragma unroll
  for (int st = 0; st < XS; ++st)
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[st][i] = load16(rX, xoff(st) + i * 32);
  __syncthreads();
  static_assert(XS % 2 == 0, "LDS buffer of a step follows from st");
  for (int k0 = 0; k0 < nk; k0 += XS) {
#pragma unroll
    for (int st = 0; st < XS; ++st) {
      const int ks = k0 + st;
      if (ks >= nk) break;
      const int buf = st & 1;   // == ks & 1
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8_t A, B0, B1, B2;
        __builtin_memcpy(&A, &xr[st][j], 16);
        const uint4 b0 = *reinterpret_cast<const uint4*>(&sW[buf][m * kKpPitch + j * 8 + kg * 4]);
        const uint4 b1 = *reinterpret_cast<const uint4*>(&sW[buf][(32 + m) * kKpPitch + j * 8 + kg * 4]);
        __builtin_memcpy(&B0, &b0, 16);
        __builtin_memcpy(&B1, &b1, 16);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B1, acc1, 0, 0, 0);
        if (gate) {
          const uint4 b2 = *reinterpret_cast<const uint4*>(&sW[buf][(64 + m) * kKpPitch + j * 8 + kg * 4]);
          __builtin_memcpy(&B2, &b2, 16);
          acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B2, acc2, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[st][i] = load16(rX, xoff(ks + XS) + i * 32);
      __syncthreads();
    }
  }
  keyproj_epilogue(acc0, acc1, acc2, a.gamma_k, a.khat + (size_t)bb * a.kh_stride,
                   gate ? a.gate + (size_t)bb * a.W * a.H_I : nullptr, a.L, a.W, a.H_I, a.eps, gate, t0, m, kg);
}

// ------------------------------------------------------------------ A1: keys, fp32 FMA
template <typename T>
__global__ __launch_bounds__(256) void keyproj_valu_kernel(IndexArgs a) {
  // block: 16 tokens; thread -> (token, output) pairs
  const int bb = blockIdx.y, t0 = blockIdx.x * 16;
  __shared__ float sk[16][64];
  const T* X = reinterpret_cast<const T*>(a.X) + (size_t)bb * a.L * a.D;
  const T* Wk = reinterpret_cast<const T*>(a.W_kI);
  for (int o = threadIdx.x; o < 16 * a.d_I; o += 256) {
    const int tt = o / a.d_I, n = o % a.d_I, t = t0 + tt;
    float s = 0.f;
    if (t < a.L)
      for (int k = 0; k < a.D; ++k) s = fmaf(load_scalar<T>(X + (size_t)t * a.D + k), load_scalar<T>(Wk + (size_t)n * a.D + k), s);
    sk[tt][n] = s;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int tt = wave; tt < 16; tt += 4) {
    const int t = t0 + tt;
    const float x = lane < a.d_I ? sk[tt][lane] : 0.f;
    const float ss = wave_sum(x * x);
    const float r = rsqrtf(ss / a.d_I + a.eps);
    if (t < a.L && lane < a.d_I) a.khat[(size_t)bb * a.kh_stride + (size_t)t * a.d_I + lane] = a.gamma_k[lane] * x * r;
  }
}

// ------------------------------------------------------------------ A2: queries and gates
// Block: QB window queries of one sequence, so every W_g / W_qI element read from L2 serves
// QB queries.  x and q of the QB queries sit in LDS in their storage type; weights stream
// in 16-byte vectors (8 bf16 or 4 fp32 per lane).
constexpr int kQB = 2;

template <typename T>
__global__ __launch_bounds__(256) void query_kernel(IndexArgs a) {
  constexpr int EPL = Vec16<T>::N;
  const int s0 = blockIdx.x * kQB, bb = blockIdx.y;
  const int nq = min(kQB, a.W - s0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  extern __shared__ float smem[];
  float* sqi = smem;                         // [QB][H_I * d_I]
  float* sg = sqi + kQB * a.H_I * a.d_I;     // [QB][H_I]
  T* sx = reinterpret_cast<T*>(smem + ((kQB * (a.H_I * a.d_I + a.H_I) + 3) & ~3));   // [QB][D], 16-byte aligned
  T* sq = sx + kQB * a.D;                    // [QB][H_q * d]
  const int qd = a.H_q * a.d;
  for (int j = 0; j < kQB; ++j) {
    const int s = min(s0 + j, a.W - 1);
    const T* xs = reinterpret_cast<const T*>(a.X) + ((size_t)bb * a.L + a.L - a.W + s) * a.D;
    const T* qs = reinterpret_cast<const T*>(a.Qwin) + ((size_t)bb * a.W + s) * qd;
    for (int i = tid * EPL; i < a.D; i += 256 * EPL)
      *reinterpret_cast<uint4*>(sx + j * a.D + i) = *reinterpret_cast<const uint4*>(xs + i);
    for (int i = tid * EPL; i < qd; i += 256 * EPL)
      *reinterpret_cast<uint4*>(sq + j * qd + i) = *reinterpret_cast<const uint4*>(qs + i);
  }
  __syncthreads();
  // gates: one wave per head, lanes over D in 16-byte vectors
  const T* Wg = reinterpret_cast<const T*>(a.W_g);
  for (int h = wave; h < a.H_I; h += 4) {
    float acc[kQB] = {};
    for (int k = lane * EPL; k < a.D; k += 64 * EPL) {
      float w[EPL];
      Vec16<T>::load(Wg + (size_t)h * a.D + k, w);
#pragma unroll
      for (int j = 0; j < kQB; ++j) {
        float xv[EPL];
        Vec16<T>::load(sx + j * a.D + k, xv);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j] = fmaf(w[e], xv[e], acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < kQB; ++j) {
      const float t = wave_sum(acc[j]);
      if (lane == 0) sg[j * a.H_I + h] = sigmoid_f(t);
    }
  }
  // down-projection: LPR lanes per W_qI row (16 bytes each), 64 / LPR rows per instruction
  const T* Wq = reinterpret_cast<const T*>(a.W_qI);
  const int LPR = a.d / EPL;                 // 16 (bf16, d = 128) .. 8 (bf16 d = 64 / f32 d = 128)
  const int rpi = 64 / LPR;
  const int sub = lane % LPR, grp = lane / LPR;
  const int nout = a.H_I * a.d_I;
  for (int o0 = wave * rpi; o0 < nout; o0 += 4 * rpi) {
    const int o = o0 + grp;
    float acc[kQB] = {};
    if (o < nout) {
      const int h = o / a.d_I;
      const int c = (h * a.H_q) / a.H_I;
      float w[EPL];
      Vec16<T>::load(Wq + (size_t)o * a.d + sub * EPL, w);
#pragma unroll
      for (int j = 0; j < kQB; ++j) {
        float qv[EPL];
        Vec16<T>::load(sq + j * qd + c * a.d + sub * EPL, qv);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j] = fmaf(w[e], qv[e], acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < kQB; ++j) {
      float t = acc[j];
      for (int msk = 1; msk < LPR; msk <<= 1) t += __shfl_xor(t, msk);
      if (o < nout && sub == 0) sqi[j * nout + o] = t;
    }
  }
  __syncthreads();
  // RMSNorm per (query, head), gate, 1/sqrt(d_I)
  const float isd = rsqrtf((float)a.d_I);
  for (int jh = wave; jh < nq * a.H_I; jh += 4) {
    const int j = jh / a.H_I, h = jh % a.H_I;
    const float x = lane < a.d_I ? sqi[j * nout + h * a.d_I + lane] : 0.f;
    const float ss = wave_sum(x * x);
    const float r = rsqrtf(ss / a.d_I + a.eps);
    float* out = a.qt + ((size_t)bb * a.W + s0 + j) * nout;
    if (lane < a.d_I) out[h * a.d_I + lane] = sg[j * a.H_I + h] * a.gamma_q[lane] * x * r * isd;
  }
}

// ------------------------------------------------------------------ A2: queries, matrix cores
// bf16, d = 128, d_I = 64, W % 32 == 0.  One wave per (sequence, indexer head h, 32 window
// queries): Q [32 x 128] of model head c(h) times W_qI[h]^T [128 x 64] on
// v_mfma_f32_32x32x16_bf16; then RMSNorm over d_I per query, the gate from the key kernel
// and 1/sqrt(d_I).  A grid of one-wave blocks spreads this latency-bound step over the chip;
// every load (operands and the 16 gates) goes out before the first wait.
__global__ __launch_bounds__(64) void query_mfma_kernel(IndexArgs a) {
  const int lane = threadIdx.x;
  const int h = blockIdx.x, mt = blockIdx.y, bb = blockIdx.z;
  const int m = lane & 31, kg = lane >> 5;
  const int c = (h * a.H_q) / a.H_I;
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.Qwin) + (size_t)bb * a.W * a.H_q * 128 + (size_t)c * 128;
  const uint16_t* Wq = reinterpret_cast<const uint16_t*>(a.W_qI) + (size_t)h * 64 * 128;
  const float isd = 0.125f;   // 1/sqrt(64)
  uint4 qa[8], wb0[8], wb1[8];
  const int s = mt * 32 + m;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    qa[j] = *reinterpret_cast<const uint4*>(Q + (size_t)s * a.H_q * 128 + j * 16 + kg * 8);
    wb0[j] = *reinterpret_cast<const uint4*>(Wq + (size_t)m * 128 + j * 16 + kg * 8);
    wb1[j] = *reinterpret_cast<const uint4*>(Wq + (size_t)(32 + m) * 128 + j * 16 + kg * 8);
  }
  float gt[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int sq = mt * 32 + 8 * (j / 4) + 4 * kg + (j % 4);
    gt[j] = a.gate[((size_t)bb * a.W + sq) * a.H_I + h];
  }
  const float gk0 = a.gamma_q[m], gk1 = a.gamma_q[32 + m];
  f32x16_t acc0 = {}, acc1 = {};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    bf16x8_t A, B0, B1;
    __builtin_memcpy(&A, &qa[j], 16);
    __builtin_memcpy(&B0, &wb0[j], 16);
    __builtin_memcpy(&B1, &wb1[j], 16);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B0, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B1, acc1, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int sq = mt * 32 + 8 * (j / 4) + 4 * kg + (j % 4);
    float ss = acc0[j] * acc0[j] + acc1[j] * acc1[j];
    ss = group_sum<32>(ss);
    const float r = rsqrtf(ss * (1.f / 64.f) + a.eps);
    float* out = a.qt + (((size_t)bb * a.W + sq) * a.H_I + h) * 64;
    out[m] = gt[j] * gk0 * acc0[j] * r * isd;
    out[32 + m] = gt[j] * gk1 * acc1[j] * r * isd;
  }
}

// ------------------------------------------------------------------ A3: scores, matrix cores
constexpr int kQPitch = 36;   // words per LDS row: 64 fp16 + 8 pad

__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)((x - (float)hi) * 2048.f);
}

// Window queries are staged kSQ at a time (split fp16 hi + lo, double-buffered in dynamic LDS),
// so the block synchronises once per kSQ queries instead of once per query.
constexpr int kSQ = 4;
constexpr int kSQWords = 32 * kQPitch;                                   // one operand plane
constexpr size_t kScoreLds = (size_t)2 * kSQ * 2 * kSQWords * sizeof(uint32_t);   // 73,728 B

// grid (ceil(L / 512), b, parts): block z of a (key block, sequence) scores its keys against
// the z-th of `parts` contiguous runs of the window's query groups and writes the running max
// to a.I + z b L; the max over the parts is the importance (exact in any order).
__global__ __launch_bounds__(512) void score_mfma_kernel(IndexArgs a) {
  // block: 512 keys (8 waves x 2 tiles x 32); H_I = 32, d_I = 64
  extern __shared__ uint32_t sQd[];   // [buf][query][hi/lo][head row * kQPitch]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bb = blockIdx.y;
  const int ng = (a.W + kSQ - 1) / kSQ;
  const int gb = (int)(blockIdx.z * (unsigned)ng / gridDim.z), ge = (int)((blockIdx.z + 1) * (unsigned)ng / gridDim.z);
  const int kbase = blockIdx.x * 512 + wave * 64;
  const int m = lane & 31, kg = lane >> 5;

  // B operands (keys): tile nt, k-step ks: lane holds k_hat[key][ks*16 + kg*8 .. +8]
  f16x8_t bh[2][4], bl[2][4];
  const float* kh = a.khat + (size_t)bb * a.L * 64;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int key = min(kbase + nt * 32 + m, a.L - 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float4 v0 = *reinterpret_cast<const float4*>(kh + (size_t)key * 64 + ks * 16 + kg * 8);
      const float4 v1 = *reinterpret_cast<const float4*>(kh + (size_t)key * 64 + ks * 16 + kg * 8 + 4);
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        _Float16 h, l;
        split_f16(v[e], h, l);
        bh[nt][ks][e] = h;
        bl[nt][ks][e] = l;
      }
    }
  }
  // query staging: a query is 32 heads x 64 dims fp32 = 512 float4, one per thread; a group
  // of kSQ queries is kSQ float4 per thread (queries past the window repeat the last one and
  // are never used)
  const float* qbase = a.qt + (size_t)bb * a.W * 2048;
  float4 pf[kSQ];
  auto fetch = [&](int g0) {
#pragma unroll
    for (int r = 0; r < kSQ; ++r)
      pf[r] = *reinterpret_cast<const float4*>(qbase + (size_t)min(g0 + r, a.W - 1) * 2048 + tid * 4);
  };
  auto stage = [&](int buf) {
    const int row = (tid * 4) >> 6, col = (tid * 4) & 63;
#pragma unroll
    for (int r = 0; r < kSQ; ++r) {
      _Float16 h[4], l[4];
      split_f16(pf[r].x, h[0], l[0]); split_f16(pf[r].y, h[1], l[1]);
      split_f16(pf[r].z, h[2], l[2]); split_f16(pf[r].w, h[3], l[3]);
      uint2 hw, lw;
      __builtin_memcpy(&hw, h, 8);
      __builtin_memcpy(&lw, l, 8);
      uint32_t* q = sQd + (size_t)((buf * kSQ + r) * 2) * kSQWords;
      *reinterpret_cast<uint2*>(&q[row * kQPitch + col / 2]) = hw;
      *reinterpret_cast<uint2*>(&q[kSQWords + row * kQPitch + col / 2]) = lw;
    }
  };
  float best0 = -INFINITY, best1 = -INFINITY;
  fetch(gb * kSQ);
  stage(0);
  __syncthreads();
  for (int gi = gb; gi < ge; ++gi) {
    const int buf = (gi - gb) & 1, g0 = gi * kSQ;
    if (gi + 1 < ge) fetch(g0 + kSQ);
    const int nq = min(kSQ, a.W - g0);
    // A operands (query heads x dims, hi and lo) of query r are read from LDS while the
    // epilogue of query r - 1 runs
    auto read_a = [&](int r, f16x8_t (&Ah)[4], f16x8_t (&Al)[4]) {
      const uint32_t* qh = sQd + (size_t)((buf * kSQ + r) * 2) * kSQWords;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 ah = *reinterpret_cast<const uint4*>(&qh[m * kQPitch + ks * 8 + kg * 4]);
        const uint4 al = *reinterpret_cast<const uint4*>(&qh[kSQWords + m * kQPitch + ks * 8 + kg * 4]);
        __builtin_memcpy(&Ah[ks], &ah, 16);
        __builtin_memcpy(&Al[ks], &al, 16);
      }
    };
    // One key tile of one query: 12 MFMAs into c = hi.hi and x = hi.lo' + lo'.hi; and its
    // epilogue: rows = heads, column = key; relu, head sum (in-lane over 16 rows, then the
    // other half-wave's 16 via a lane swap), causal mask, running max.
    auto mfma_tile = [&](int t, const f16x8_t (&Ah)[4], const f16x8_t (&Al)[4], f32x16_t& c, f32x16_t& x) {
      c = x = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ah[ks], bh[t][ks], c, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ah[ks], bl[t][ks], x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_32x32x16_f16(Al[ks], bh[t][ks], x, 0, 0, 0);
      }
    };
    auto epi_tile = [&](int t, int r, const f32x16_t& c, const f32x16_t& x, float& best) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) sum += fmaxf(fmaf(x[j], 1.f / 2048.f, c[j]), 0.f);
      const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum), false, false);
      sum = __uint_as_float(w[0]) + __uint_as_float(w[1]);
      if (kbase + t * 32 + m <= a.L - a.W + g0 + r) best = fmaxf(best, sum);
    };
    // interleave: one MFMA, then 4 VALU of the epilogue running beside it
    auto interleave = [&]() {
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    };
    f16x8_t Ah[4], Al[4];
    f32x16_t c0, x0, c1, x1;
    if (nq == kSQ) {
      // software-pipelined over the two key tiles: tile 1's MFMAs of query r run beside
      // tile 0's epilogue of r, and tile 0's MFMAs of r + 1 beside tile 1's epilogue of r,
      // so the matrix core and the VALU work at the same time
      read_a(0, Ah, Al);
      mfma_tile(0, Ah, Al, c0, x0);
#pragma unroll
      for (int r = 0; r < kSQ; ++r) {
        mfma_tile(1, Ah, Al, c1, x1);
        epi_tile(0, r, c0, x0, best0);
        interleave();
        if (r + 1 < kSQ) {
          read_a(r + 1, Ah, Al);
          mfma_tile(0, Ah, Al, c0, x0);
        }
        epi_tile(1, r, c1, x1, best1);
        if (r + 1 < kSQ) {
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // the DS reads of query r + 1
          interleave();
        }
      }
    } else {
      for (int r = 0; r < nq; ++r) {
        read_a(r, Ah, Al);
        mfma_tile(0, Ah, Al, c0, x0);
        mfma_tile(1, Ah, Al, c1, x1);
        epi_tile(0, r, c0, x0, best0);
        epi_tile(1, r, c1, x1, best1);
      }
    }
    if (gi + 1 < ge) stage(buf ^ 1);
    __syncthreads();
  }
  float* Ir = a.I + ((size_t)blockIdx.z * a.b + bb) * a.L;
  if (kg == 0) {
    if (kbase + m < a.L) Ir[kbase + m] = best0;
    if (kbase + 32 + m < a.L) Ir[kbase + 32 + m] = best1;
  }
}

// ------------------------------------------------------------------ A3: scores, fp32 FMA
__global__ __launch_bounds__(256) void score_valu_kernel(IndexArgs a) {
  // block: 256 keys, one per thread; queries staged per window position in LDS
  const int bb = blockIdx.y, t = blockIdx.x * 256 + threadIdx.x;
  extern __shared__ float sq[];   // [H_I * d_I]
  float k[64];
  const int tt = min(t, a.L - 1);
#pragma unroll
  for (int i = 0; i < 64; ++i) k[i] = i < a.d_I ? a.khat[((size_t)bb * a.L + tt) * a.d_I + i] : 0.f;
  float best = -INFINITY;
  const int nq = a.H_I * a.d_I;
  for (int s = 0; s < a.W; ++s) {
    __syncthreads();
    for (int i = threadIdx.x; i < nq; i += 256) sq[i] = a.qt[((size_t)bb * a.W + s) * nq + i];
    __syncthreads();
    float A = 0.f;
    for (int h = 0; h < a.H_I; ++h) {
      float x = 0.f;
#pragma unroll
      for (int i = 0; i < 64; ++i)
        if (i < a.d_I) x = fmaf(sq[h * a.d_I + i], k[i], x);
      A += fmaxf(x, 0.f);
    }
    if (t <= a.L - a.W + s) best = fmaxf(best, A);
  }
  if (t < a.L) a.I[(size_t)bb * a.L + t] = best;
}

// Window splits of the score launch: one unless the (key block, sequence) grid leaves CUs
// idle; then enough runs of query groups to give every CU a block.
static int score_parts(int b, int Ls, int W, int H_I, int d_I) {
  if (H_I != 32 || d_I != 64) return 1;
  const long long blocks = (long long)b * ((Ls + 511) / 512);
  const int ng = (W + kSQ - 1) / kSQ;
  if (blocks >= kFillBlocks) return 1;
  return (int)std::min<long long>(ng, (kFillBlocks + blocks - 1) / blocks);
}

// Max over `parts` partial importances [parts][n] -> I [n] (NaN if any part is NaN).
__global__ __launch_bounds__(256) void part_max_kernel(float* I, const float* part, int parts, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float m = part[i];
  for (int z = 1; z < parts; ++z) {
    const float c = part[(size_t)z * n + i];
    m = (m != m || c != c) ? NAN : fmaxf(m, c);
  }
  I[i] = m;
}

// The indexer's launches: keys (and, on the matrix-core path, the window's gate logits) over
// a.L tokens of X into a.khat (stride a.kh_stride), the window queries, then the window's
// scores against Ls keys from khat_s (stride Ls d_I) into I, as `parts` partial maxima
// [parts][b][Ls] (score_parts of the same shape).
static kvm_status index_launch(IndexArgs a, float* gate_ws, bool bf, const float* khat_s, int Ls, float* I,
                               int parts, hipStream_t s) {
  // matrix-core path: bf16, d_I = 64, H_I <= 32, d = 128, D % 64 == 0, W % 32 == 0
  const bool mfma = bf && a.d_I == 64 && a.H_I <= 32 && a.d == 128 && a.D % 64 == 0 && a.W % 32 == 0;
  a.gate = mfma ? gate_ws : nullptr;
  const size_t qsmem = (size_t)((kQB * (a.H_I * a.d_I + a.H_I) + 3) & ~3) * sizeof(float) +
                       (size_t)kQB * (a.D + a.H_q * a.d) * (bf ? 2 : 4);
  // the streaming variant addresses its buffers with 32-bit byte offsets (64 D 2 bytes of
  // weights): wide models fall back to the wide-grid kernel
  if (mfma && ((long long)a.b * ((a.L + kKpTB - 1) / kKpTB) >= kFillBlocks || a.D > (1 << 20)))
    hipLaunchKernelGGL(keyproj_mfma_kernel, dim3((a.L + kKpTB - 1) / kKpTB, a.b), dim3(kKpNW * 64), 0, s, a);
  else if (mfma && (long long)a.b * ((a.L + kKpsNW * 32 - 1) / (kKpsNW * 32)) >= kFillBlocks)
    hipLaunchKernelGGL((keyproj_stream_kernel<kKpsNW, kKpsXS, kKpsWD>), dim3((a.L + kKpsNW * 32 - 1) / (kKpsNW * 32), a.b),
                       dim3((kKpsNW + 1) * 64), 0, s, a);
  else if (mfma)   // smaller still (batch 1): 2 compute waves per block, twice the blocks
    hipLaunchKernelGGL((keyproj_stream_kernel<2, kKpsXS, kKpsWD>), dim3((a.L + 63) / 64, a.b), dim3(3 * 64), 0, s, a);
  else if (bf)
    hipLaunchKernelGGL(keyproj_valu_kernel<uint16_t>, dim3((a.L + 15) / 16, a.b), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(keyproj_valu_kernel<float>, dim3((a.L + 15) / 16, a.b), dim3(256), 0, s, a);
  const dim3 qgrid((a.W + kQB - 1) / kQB, a.b);
  if (mfma)
    hipLaunchKernelGGL(query_mfma_kernel, dim3(a.H_I, a.W / 32, a.b), dim3(64), 0, s, a);
  else if (bf)
    hipLaunchKernelGGL(query_kernel<uint16_t>, qgrid, dim3(256), qsmem, s, a);
  else
    hipLaunchKernelGGL(query_kernel<float>, qgrid, dim3(256), qsmem, s, a);
  a.khat = const_cast<float*>(khat_s);
  a.L = Ls;
  a.I = I;
  if (a.H_I == 32 && a.d_I == 64) {
    static bool lds_set = false;   // a function attribute: setting it once per process suffices
    if (!lds_set) {
      const kvm_status st = check_hip(hipFuncSetAttribute(reinterpret_cast<const void*>(&score_mfma_kernel),
                                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kScoreLds),
                                      "score kernel LDS size");
      if (st != KVM_OK) return st;
      lds_set = true;
    }
    hipLaunchKernelGGL(score_mfma_kernel, dim3((Ls + 511) / 512, a.b, parts), dim3(512), kScoreLds, s, a);
  } else {
    hipLaunchKernelGGL(score_valu_kernel, dim3((Ls + 255) / 256, a.b), dim3(256),
                       (size_t)a.H_I * a.d_I * sizeof(float), s, a);
  }
  return KVM_OK;
}

struct IndexWs { size_t kh, qt, gate, part, total; int parts; };
static IndexWs index_ws(const kvm_index_desc* d) {
  IndexWs w;
  w.parts = score_parts(d->b, d->L, d->W, d->H_I, d->d_I);
  w.kh = 0;
  w.qt = align_up(w.kh + (size_t)d->b * d->L * d->d_I * sizeof(float), 256);
  w.gate = align_up(w.qt + (size_t)d->b * d->W * d->H_I * d->d_I * sizeof(float), 256);
  w.part = align_up(w.gate + (size_t)d->b * d->W * d->H_I * sizeof(float), 256);
  const size_t part_bytes = w.parts > 1 ? (size_t)w.parts * d->b * d->L * sizeof(float) : 0;
  w.total = align_up(w.part + part_bytes, 256);
  return w;
}

}  // namespace kvm

using namespace kvm;

extern "C" size_t kvm_index_workspace_size(const kvm_index_desc* d) {
  if (!d || d->b <= 0 || d->L <= 0 || d->d_I <= 0 || d->W <= 0 || d->H_I <= 0) return 0;
  return index_ws(d).total;
}

extern "C" kvm_status kvm_index_score(const kvm_index_desc* d, const void* X, const void* Qwin, const void* W_kI,
                                      const float* gamma_k, const void* W_qI, const float* gamma_q, const void* W_g,
                                      float* I, float* khat, void* ws, size_t ws_bytes, void* stream) {
  KVM_PTR(d);
  KVM_REQUIRE(d->b > 0 && d->L > 0 && d->D > 0 && d->H_q > 0 && d->H_I > 0, KVM_ERR_SHAPE,
              "b, L, D, H_q, H_I must be positive");
  KVM_REQUIRE(d->d_I == 32 || d->d_I == 64, KVM_ERR_SHAPE, "d_I %d not in {32, 64}", d->d_I);
  KVM_REQUIRE(d->d == 64 || d->d == 128, KVM_ERR_SHAPE, "head dim %d not in {64, 128}", d->d);
  KVM_REQUIRE(d->D % 8 == 0, KVM_ERR_SHAPE, "D %% 8 != 0");
  KVM_REQUIRE(d->W >= 1 && d->W <= d->L, KVM_ERR_RANGE, "window %d outside [1, L]", d->W);
  KVM_REQUIRE(d->dtype == KVM_F32 || d->dtype == KVM_BF16, KVM_ERR_DTYPE, "dtype %d", d->dtype);
  KVM_PTR_ALIGNED(X); KVM_PTR_ALIGNED(Qwin); KVM_PTR_ALIGNED(W_kI); KVM_PTR_ALIGNED(gamma_k);
  KVM_PTR_ALIGNED(W_qI); KVM_PTR_ALIGNED(gamma_q); KVM_PTR_ALIGNED(W_g); KVM_PTR_ALIGNED(I);
  KVM_OPT_ALIGNED(khat);
  const IndexWs w = index_ws(d);
  KVM_REQUIRE(ws != nullptr && ws_bytes >= w.total, KVM_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  KVM_ALIGNED(ws);
  const size_t esz = d->dtype == KVM_BF16 ? 2 : 4;
  const size_t qsmem = (size_t)((kQB * (d->H_I * d->d_I + d->H_I) + 3) & ~3) * sizeof(float) +
                       (size_t)kQB * (d->D + d->H_q * d->d) * esz;
  KVM_REQUIRE(qsmem <= 64 * 1024, KVM_ERR_SHAPE, "D + H_q*d too large for the query kernel");
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;

  IndexArgs a{};
  a.X = X; a.Qwin = Qwin; a.W_kI = W_kI; a.gamma_k = gamma_k; a.W_qI = W_qI; a.gamma_q = gamma_q; a.W_g = W_g;
  a.I = I;
  char* base = static_cast<char*>(ws);
  a.khat = khat ? khat : reinterpret_cast<float*>(base + w.kh);
  a.qt = reinterpret_cast<float*>(base + w.qt);
  a.b = d->b; a.L = d->L; a.D = d->D; a.H_q = d->H_q; a.d = d->d; a.H_I = d->H_I; a.d_I = d->d_I; a.W = d->W;
  a.eps = d->eps_rms;
  a.kh_stride = (size_t)d->L * d->d_I;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* part = w.parts > 1 ? reinterpret_cast<float*>(base + w.part) : I;
  st = index_launch(a, reinterpret_cast<float*>(base + w.gate), d->dtype == KVM_BF16, a.khat, d->L, part, w.parts, s);
  if (st != KVM_OK) return st;
  if (w.parts > 1) {
    const size_t n = (size_t)d->b * d->L;
    hipLaunchKernelGGL(part_max_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, I, part, w.parts, n);
  }
  return check_hip(hipGetLastError(), "index kernels launch");
}

// ------------------------------------------------------------------ chunked pre-eviction
namespace kvm {

// grid (ceil(max(C H_kv D / 8, C) / 256), b), 256 threads: the chunk's token-major K, V rows
// into the pool's head-major rows P .. P + C - 1 (16 bytes per thread; skipped when K is
// NULL: the rows are already there), and their positions.
template <typename T>
__global__ __launch_bounds__(256) void chunk_append_kernel(const T* K, const T* V, T* Kp, T* Vp, int32_t* pos,
                                                           int C, int H_kv, int D, int P, int Lv, int start) {
  constexpr int N = 16 / sizeof(T);
  const int bb = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;          // 16-byte chunk of the batch row's C x H_kv x D
  const int per_tok = H_kv * D / N;
  if (K && i < C * per_tok) {
    const int t = i / per_tok, r = i % per_tok, g = r / (D / N), c = (r % (D / N)) * N;
    const size_t src = (((size_t)bb * C + t) * H_kv + g) * D + c;
    const size_t dst = (((size_t)bb * H_kv + g) * Lv + P + t) * D + c;
    *reinterpret_cast<uint4*>(Kp + dst) = *reinterpret_cast<const uint4*>(K + src);
    *reinterpret_cast<uint4*>(Vp + dst) = *reinterpret_cast<const uint4*>(V + src);
  }
  if (i < C) pos[(size_t)bb * Lv + P + i] = start + i;
}

// grid (ceil(Lv / 256), b): a pooled key keeps the running max of its importance (NaN
// propagates); a chunk key takes this window's.
__global__ __launch_bounds__(256) void chunk_max_kernel(float* I, const float* Icur, int parts, int b, int P, int Lv) {
  const int t = blockIdx.x * 256 + threadIdx.x, bb = blockIdx.y;
  if (t >= Lv) return;
  const size_t i = (size_t)bb * Lv + t;
  float c = Icur[i];
  for (int z = 1; z < parts; ++z) {
    const float x = Icur[(size_t)z * b * Lv + i];
    c = (c != c || x != x) ? NAN : fmaxf(c, x);
  }
  if (t < P) {
    const float o = I[i];
    I[i] = (o != o || c != c) ? NAN : fmaxf(o, c);
  } else {
    I[i] = c;
  }
}

// One thread per (row, token, word) of the kept tokens' side data, words 0 .. d_I-1 the
// indexer key, d_I the importance, d_I+1 the position: each into the token's slot of the next
// pool (slot_map; tokens without a slot in [0, cap) are dropped).  Absent outputs are skipped.
__global__ __launch_bounds__(256) void chunk_side_kernel(const float* khat_p, const float* I_p, const int32_t* pos_p,
                                                         const int32_t* smap, float* khat_n, float* I_n,
                                                         int32_t* pos_n, int rows, int Lv, int cap, int d_I) {
  const int words = d_I + 2;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)rows * Lv * words) return;
  const size_t rt = i / words;
  const int w = (int)(i % words);
  const int slot = smap[rt];
  if (slot < 0 || slot >= cap) return;
  const size_t dst = (size_t)(rt / Lv) * cap + slot;
  if (w < d_I) {
    if (khat_n) khat_n[dst * d_I + w] = khat_p[rt * d_I + w];
  } else if (w == d_I) {
    if (I_n) I_n[dst] = I_p[rt];
  } else if (pos_n) {
    pos_n[dst] = pos_p[rt];
  }
}

struct ChunkWs { size_t idx, qt, gate, icur, ids, smap, comp, total; };
static ChunkWs chunk_ws(const kvm_chunk_desc* d, size_t comp_bytes) {
  const size_t Lv = (size_t)d->P + d->C;
  const kvm_topk_desc td{d->b, (int32_t)Lv, d->B, d->R, d->recent_inclusive};
  const int keep = kvm_topk_keep(&td);
  ChunkWs w;
  w.idx = 0;
  w.qt = 0;
  w.gate = align_up(w.qt + (size_t)d->b * d->W * d->H_I * d->d_I * sizeof(float), 256);
  w.icur = align_up(w.gate + (size_t)d->b * d->W * d->H_I * sizeof(float), 256);
  w.ids = align_up(w.icur + (size_t)score_parts(d->b, (int)Lv, d->W, d->H_I, d->d_I) * d->b * Lv * sizeof(float), 256);
  w.smap = align_up(w.ids + (size_t)d->b * (keep > 0 ? keep : 1) * sizeof(int32_t), 256);
  w.comp = align_up(w.smap + (size_t)d->b * Lv * sizeof(int32_t), 256);
  w.total = align_up(w.comp + comp_bytes, 256);
  return w;
}

static kvm_compact_desc chunk_compact_desc(const kvm_chunk_desc* d, int keep) {
  kvm_compact_desc c{};
  c.b = d->b; c.L = d->P + d->C; c.H_kv = d->H_kv; c.d = d->d; c.cap = d->cap_out; c.keep = keep;
  c.dtype = d->dtype; c.per_head = 0; c.kv_head_major = 1; c.flags = KVM_FUSE_MEM; c.lam = d->lam;
  c.v_row_major = d->final ? 0 : 1;
  return c;
}

}  // namespace kvm

extern "C" int32_t kvm_chunk_keep(const kvm_chunk_desc* d) {
  if (!d) return -1;
  const kvm_topk_desc td{d->b, d->P + d->C, d->B, d->R, d->recent_inclusive};
  return kvm_topk_keep(&td);
}

extern "C" size_t kvm_chunk_workspace_size(const kvm_chunk_desc* d) {
  if (!d || d->b <= 0 || d->C <= 0 || d->P < 0 || d->W <= 0 || d->H_I <= 0 || d->d_I <= 0) return 0;
  const int keep = kvm_chunk_keep(d);
  if (keep < 0) return 0;
  const kvm_compact_desc cd = chunk_compact_desc(d, keep);
  return chunk_ws(d, kvm_compact_workspace_size(&cd)).total;
}

extern "C" kvm_status kvm_index_evict_chunk(const kvm_chunk_desc* d, const void* X, const void* Qwin, const void* K,
                                            const void* V, const void* W_kI, const float* gamma_k, const void* W_qI,
                                            const float* gamma_q, const void* W_g, void* Kp, void* Vp, float* khat_p,
                                            float* I_p, int32_t* pos_p, void* Kn, void* Vn, float* khat_n,
                                            float* I_n, int32_t* pos_n, float* M, float* bvec, void* ws,
                                            size_t ws_bytes, void* stream) {
  KVM_PTR(d);
  KVM_REQUIRE(d->b > 0 && d->D > 0 && d->H_q > 0 && d->H_kv > 0 && d->H_I > 0 && d->C > 0 && d->P >= 0,
              KVM_ERR_SHAPE, "b, D, H_q, H_kv, H_I, C must be positive and P >= 0");
  KVM_REQUIRE(d->d_I == 32 || d->d_I == 64, KVM_ERR_SHAPE, "d_I %d not in {32, 64}", d->d_I);
  KVM_REQUIRE(d->d == 64 || d->d == 128, KVM_ERR_SHAPE, "head dim %d not in {64, 128}", d->d);
  KVM_REQUIRE(d->D % 8 == 0, KVM_ERR_SHAPE, "D %% 8 != 0");
  KVM_REQUIRE(d->H_q % d->H_kv == 0, KVM_ERR_SHAPE, "H_q %d not a multiple of H_kv %d", d->H_q, d->H_kv);
  KVM_REQUIRE(d->dtype == KVM_F32 || d->dtype == KVM_BF16, KVM_ERR_DTYPE, "dtype %d", d->dtype);
  KVM_REQUIRE(d->W >= 1 && d->W <= d->C && d->R >= 0 && d->R <= d->C, KVM_ERR_RANGE,
              "the chunk (%d tokens) must hold the window %d and the recent window %d", d->C, d->W, d->R);
  KVM_REQUIRE(d->lam >= 0.f && d->lam <= 1.f, KVM_ERR_RANGE, "lam %g outside [0, 1]", d->lam);
  const int keep = kvm_chunk_keep(d);
  KVM_REQUIRE(keep >= 0, KVM_ERR_RANGE, "budget %d below the recent window %d", d->B, d->R);
  KVM_REQUIRE(d->cap_out >= keep, KVM_ERR_RANGE, "cap_out %d below the kept %d", d->cap_out, keep);
  KVM_REQUIRE((K == nullptr) == (V == nullptr), KVM_ERR_NULL, "K and V must both be given or both NULL (in place)");
  KVM_PTR_ALIGNED(X); KVM_PTR_ALIGNED(Qwin); KVM_OPT_ALIGNED(K); KVM_OPT_ALIGNED(V); KVM_PTR_ALIGNED(W_kI);
  KVM_PTR_ALIGNED(gamma_k); KVM_PTR_ALIGNED(W_qI); KVM_PTR_ALIGNED(gamma_q); KVM_PTR_ALIGNED(W_g);
  KVM_PTR_ALIGNED(Kp); KVM_PTR_ALIGNED(Vp); KVM_PTR_ALIGNED(khat_p); KVM_PTR_ALIGNED(I_p); KVM_PTR_ALIGNED(pos_p);
  KVM_PTR_ALIGNED(Kn); KVM_PTR_ALIGNED(Vn); KVM_PTR_ALIGNED(M); KVM_PTR_ALIGNED(bvec);
  KVM_OPT_ALIGNED(khat_n); KVM_OPT_ALIGNED(I_n); KVM_OPT_ALIGNED(pos_n);
  const size_t esz = d->dtype == KVM_BF16 ? 2 : 4;
  const size_t qsmem = (size_t)((kQB * (d->H_I * d->d_I + d->H_I) + 3) & ~3) * sizeof(float) +
                       (size_t)kQB * (d->D + d->H_q * d->d) * esz;
  KVM_REQUIRE(qsmem <= 64 * 1024, KVM_ERR_SHAPE, "D + H_q*d too large for the query kernel");
  const kvm_compact_desc cd = chunk_compact_desc(d, keep);
  const size_t cbytes = kvm_compact_workspace_size(&cd);
  const ChunkWs w = chunk_ws(d, cbytes);
  KVM_REQUIRE(ws != nullptr && ws_bytes >= w.total, KVM_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, w.total);
  KVM_ALIGNED(ws);
  kvm_status st = require_gfx950();
  if (st != KVM_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  const int Lv = d->P + d->C;
  // 1. the chunk's K, V (unless already in place: K = V = NULL) and positions join the pool
  const int nchunk16 = K ? d->C * d->H_kv * d->d / (int)(16 / esz) : 0;
  const dim3 agrid((std::max(nchunk16, d->C) + 255) / 256, d->b);
  if (d->dtype == KVM_BF16)
    hipLaunchKernelGGL(chunk_append_kernel<uint16_t>, agrid, dim3(256), 0, s, static_cast<const uint16_t*>(K),
                       static_cast<const uint16_t*>(V), static_cast<uint16_t*>(Kp), static_cast<uint16_t*>(Vp), pos_p,
                       d->C, d->H_kv, d->d, d->P, Lv, d->start);
  else
    hipLaunchKernelGGL(chunk_append_kernel<float>, agrid, dim3(256), 0, s, static_cast<const float*>(K),
                       static_cast<const float*>(V), static_cast<float*>(Kp), static_cast<float*>(Vp), pos_p,
                       d->C, d->H_kv, d->d, d->P, Lv, d->start);
  // 2. the chunk's indexer keys (into pool rows P ..), its window's queries, the window's
  //    scores against pool and chunk (in position order), the pool's running max
  IndexArgs a{};
  a.X = X; a.Qwin = Qwin; a.W_kI = W_kI; a.gamma_k = gamma_k; a.W_qI = W_qI; a.gamma_q = gamma_q; a.W_g = W_g;
  a.khat = khat_p + (size_t)d->P * d->d_I;
  a.kh_stride = (size_t)Lv * d->d_I;
  a.qt = reinterpret_cast<float*>(base + w.qt);
  a.b = d->b; a.L = d->C; a.D = d->D; a.H_q = d->H_q; a.d = d->d; a.H_I = d->H_I; a.d_I = d->d_I; a.W = d->W;
  a.eps = d->eps_rms;
  float* icur = reinterpret_cast<float*>(base + w.icur);
  const int parts = score_parts(d->b, Lv, d->W, d->H_I, d->d_I);
  st = index_launch(a, reinterpret_cast<float*>(base + w.gate), d->dtype == KVM_BF16, khat_p, Lv, icur, parts, s);
  if (st != KVM_OK) return st;
  hipLaunchKernelGGL(chunk_max_kernel, dim3((Lv + 255) / 256, d->b), dim3(256), 0, s, I_p, icur, parts, d->b, d->P,
                     Lv);
  st = check_hip(hipGetLastError(), "chunk kernels launch");
  if (st != KVM_OK) return st;
  // 3. the budget over pool and chunk, the compaction with the memory fold, the side data
  int32_t* ids = reinterpret_cast<int32_t*>(base + w.ids);
  int32_t* smap = reinterpret_cast<int32_t*>(base + w.smap);
  const kvm_topk_desc td{d->b, Lv, d->B, d->R, d->recent_inclusive};
  st = kvm_topk_select(&td, I_p, ids, smap, nullptr, 0, stream);
  if (st != KVM_OK) return st;
  st = kvm_compact_kv(&cd, Kp, Vp, smap, ids, Kn, Vn, M, bvec, nullptr, nullptr, nullptr, nullptr,
                      base + w.comp, cbytes, stream);
  if (st != KVM_OK) return st;
  if (khat_n || I_n || pos_n) {
    const size_t total = (size_t)d->b * Lv * (d->d_I + 2);
    hipLaunchKernelGGL(chunk_side_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, khat_p, I_p, pos_p,
                       smap, khat_n, I_n, pos_n, d->b, Lv, d->cap_out, d->d_I);
    st = check_hip(hipGetLastError(), "chunk side-data launch");
  }
  return st;
}
