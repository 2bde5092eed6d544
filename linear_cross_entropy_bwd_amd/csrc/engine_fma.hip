// fp32 engine: LDS-tiled FMA contractions for FLCE_F32 inputs.
//
// One output tile per 256-thread block: 64x64 (4x4 outputs per thread) for dW,
// 64x32 (4x2) for the logits and dH; K in steps of 64 staged through LDS in
// [k][m] order.  The next step's operand
// values are loaded into registers before the current step's FMAs, so their
// latency hides under the arithmetic.  Operands are described by (pointer,
// leading dimension, k-major flag): a k-major operand has its reduction index
// contiguous in memory.  The three contractions are
//   logits  Z[t, j]  = sum_k H[t, k] W[j, k]        A = H (k-major), B = W (k-major)
//   dH      dH[t, k] = sum_j G[t, j] W[j, k]        A = G (k-major), B = W (n-major)
//   dW      dW[j, k] = sum_t G[t, j] H[t, k]        A = G^T (m-major), B = H (n-major)
// fp32 inputs keep fp32 products and sums, which the fp32 tolerances need;
// each output is one fmaf chain over k in increasing order.
#include "device_util.h"
#include "flce_internal.h"

namespace flce {

namespace {

constexpr int BM = 64, BN = 64, BK = 64;
constexpr int kPad = 4;  // keeps rows 16-byte aligned for the vector fragment reads
// The logits tiles are 64 tokens x 32 vocabulary columns: small problems then
// spread over twice as many workgroups.  Their 32 columns are one statistics
// group, so the plan's fp32 group width must equal kLogitsBN.
constexpr int kLogitsBN = 32;
// dH's tile width (its tiles are 64 x kDhBN); the plan counts dH tiles the same way.
constexpr int kDhBN = kFmaDhTileCols;

// Values of one fragment row: 4 (float4) or 2 (float2) consecutive floats.
template <int W>
__device__ __forceinline__ void read_row(const float* p, float (&v)[W]) {
  static_assert(W == 4 || W == 2, "fragment rows are 2 or 4 wide");
  if constexpr (W == 4) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
    const float2 x = *reinterpret_cast<const float2*>(p);
    v[0] = x.x; v[1] = x.y;
  }
}

// Main loop of a 64 x BNT output tile (BNT = 64 or 32) per 256-thread block;
// thread (ty, tx) = (tid / 16, tid % 16) owns rows 4 ty .. 4 ty + 3 and
// columns (BNT / 16) tx .. (BNT / 16) tx + BNT / 16 - 1.
template <typename TA, typename TB, bool A_KMAJ, bool B_KMAJ, int BNT = BN>
struct TileLoop {
  static constexpr int JN = BNT / 16;

  // An operand of extent E (64 or 32) along m: each thread stages BK E / 256
  // values per step.  The lanes of a wave run along the operand's contiguous
  // index (k for a k-major operand, m otherwise), so each load instruction
  // reads consecutive values: all 64 lanes along it, or, for an m-major
  // operand of extent 32, lanes 0-31 and 32-63 on two consecutive k.  The
  // wave's other index steps from the wave number.  Loads use indices clamped
  // into the operand and are issued unconditionally; the values outside it
  // are replaced by 0 only when they are written to LDS, so nothing uses a
  // loaded value before the step that needs it.
  //   fix  = the contiguous index of lane l: l (or l % 32)
  //   step = the other index of value q: w + 4 q (or 2 w + l / 32 + 8 q)
  template <bool KMAJ, int E>
  static __device__ __forceinline__ void lane_indices(int& fix, int (&step)[BK * E / 256]) {
    static_assert(E == 64 || E == 32, "extents are 64 or 32");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr bool kPair = !KMAJ && E == 32;
    fix = kPair ? (lane & 31) : lane;
#pragma unroll
    for (int q = 0; q < BK * E / 256; ++q) step[q] = kPair ? 2 * wave + (lane >> 5) + 8 * q : wave + 4 * q;
  }

  template <bool KMAJ, int E, typename T>
  static __device__ __forceinline__ void fetch(const T* __restrict__ P, int64_t ld, int64_t M, int64_t K,
                                               int64_t m0, int64_t k0, float (&r)[BK * E / 256]) {
    int fix, step[BK * E / 256];
    lane_indices<KMAJ, E>(fix, step);
    const int64_t lim_fix = KMAJ ? K : M, lim_step = KMAJ ? M : K;
    const int64_t g_fix = (KMAJ ? k0 : m0) + fix;
    const int64_t c_fix = g_fix < lim_fix ? g_fix : lim_fix - 1;
#pragma unroll
    for (int q = 0; q < BK * E / 256; ++q) {
      const int64_t g_step = (KMAJ ? m0 : k0) + step[q];
      const int64_t c_step = g_step < lim_step ? g_step : lim_step - 1;
      r[q] = Elem<T>::ld(P, c_step * ld + c_fix);
    }
  }

  // LDS holds [k][m]: a k-major operand is transposed here.  (m0, k0) is the
  // step the values were fetched for.
  template <bool KMAJ, int E>
  static __device__ __forceinline__ void stash(float (*S)[E + kPad], const float (&r)[BK * E / 256], int64_t M,
                                               int64_t K, int64_t m0, int64_t k0) {
    int fix, step[BK * E / 256];
    lane_indices<KMAJ, E>(fix, step);
    const int64_t lim_fix = KMAJ ? K : M, lim_step = KMAJ ? M : K;
    const bool fix_in = (KMAJ ? k0 : m0) + fix < lim_fix;
#pragma unroll
    for (int q = 0; q < BK * E / 256; ++q) {
      const bool in = fix_in && (KMAJ ? m0 : k0) + step[q] < lim_step;
      const float x = in ? r[q] : 0.0f;
      if (KMAJ)
        S[fix][step[q]] = x;
      else
        S[step[q]][fix] = x;
    }
  }

  // Accumulate acc[4][JN] for the tile at (m0, n0); rows m < M, cols n < N, k < K.
  // M, N >= 1; K may be 0 (an empty vocabulary split), which leaves zeros.
  static __device__ __forceinline__ void run(const TA* __restrict__ A, int64_t lda, const TB* __restrict__ B,
                                             int64_t ldb, int64_t M, int64_t N, int64_t K, int64_t m0, int64_t n0,
                                             float (&acc)[4][JN]) {
    __shared__ __align__(16) float As[BK][BM + kPad];
    __shared__ __align__(16) float Bs[BK][BNT + kPad];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j) acc[i][j] = 0.0f;
    if (K <= 0) return;

    float ra[BK * BM / 256], rb[BK * BNT / 256];
    fetch<A_KMAJ, BM>(A, lda, M, K, m0, 0, ra);
    fetch<B_KMAJ, BNT>(B, ldb, N, K, n0, 0, rb);
    for (int64_t k0 = 0; k0 < K; k0 += BK) {
      __syncthreads();  // the previous step's fragment reads are done
      stash<A_KMAJ, BM>(As, ra, M, K, m0, k0);
      stash<B_KMAJ, BNT>(Bs, rb, N, K, n0, k0);
      __syncthreads();
      // the next step's loads (clamped, so in bounds past the end too) fly
      // under this step's FMAs
      fetch<A_KMAJ, BM>(A, lda, M, K, m0, k0 + BK, ra);
      fetch<B_KMAJ, BNT>(B, ldb, N, K, n0, k0 + BK, rb);
      // fragment reads one k ahead of the FMAs that use them
      float av[4], bv[JN];
      read_row<4>(&As[0][ty * 4], av);
      read_row<JN>(&Bs[0][tx * JN], bv);
#pragma unroll 8
      for (int kk = 0; kk < BK; ++kk) {
        const int kn = kk + 1 < BK ? kk + 1 : kk;
        float an[4], bn[JN];
        read_row<4>(&As[kn][ty * 4], an);
        read_row<JN>(&Bs[kn][tx * JN], bn);
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of this k's FMAs
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < JN; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = an[i];
#pragma unroll
        for (int j = 0; j < JN; ++j) bv[j] = bn[j];
      }
    }
  }
};

// Logits tile (rows = chunk tokens, cols = vocabulary): per-row max and
// sum-exp over the tile's kLogitsBN columns (one vocabulary group), the target
// logit, and optionally exp(z - group max) into the chunk's buffer.
// Recompute mode (lse_in != nullptr, the backward from the saved LSE): the
// buffer gets G = (exp(z - lse) - [j = y]) * scale directly, scale = upstream
// gradient times 1/n_valid (mean) or 1 (sum), 0 for ignored rows.
template <typename T>
__global__ __launch_bounds__(256) void fma_logits_kernel(const T* __restrict__ H, const T* __restrict__ W,
                                                         int64_t rows, int64_t d, int64_t v, int64_t vp,
                                                         const int64_t* __restrict__ labels, float* __restrict__ zy,
                                                         float* __restrict__ pm, float* __restrict__ ps, int64_t C,
                                                         float* __restrict__ prob, const float* __restrict__ lse_in,
                                                         const float* __restrict__ grad_out,
                                                         const int32_t* __restrict__ nvalid, int32_t reduction,
                                                         int64_t ignore_index) {
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * kLogitsBN;
  constexpr int JN = kLogitsBN / 16;  // columns per thread
  float acc[4][JN];
  TileLoop<T, T, true, true, kLogitsBN>::run(H, d, W, d, rows, v, d, m0, n0, acc);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t g = blockIdx.y;
  if (lse_in != nullptr) {
    const float go = grad_out != nullptr ? *grad_out : 1.0f;
    const int32_t nv = *nvalid;
    const float red = reduction == FLCE_SUM ? 1.0f : (nv > 0 ? 1.0f / static_cast<float>(nv) : 0.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = m0 + ty * 4 + i;
      if (t >= rows) continue;
      const int64_t y = labels[t];
      const float sc = y != ignore_index ? go * red : 0.0f;
      const float l = lse_in[t];
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        const int64_t n = n0 + tx * JN + j;
        if (n >= vp) continue;
        const float gv = n < v ? (expf(acc[i][j] - l) - (n == y ? 1.0f : 0.0f)) * sc : 0.0f;
        prob[t * vp + n] = gv;
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = m0 + ty * 4 + i;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < JN; ++j)
      if (n0 + tx * JN + j < v) mx = fmaxf(mx, acc[i][j]);
    for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float e[JN], s = 0.0f;
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      e[j] = (n0 + tx * JN + j < v) ? fast_exp(acc[i][j] - mx) : 0.0f;
      s += e[j];
    }
    for (int off = 8; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (t < rows) {
      if (tx == 0) {
        pm[g * C + t] = mx;
        ps[g * C + t] = s;
      }
      const int64_t y = labels[t];
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        const int64_t n = n0 + tx * JN + j;
        if (n == y && n < v) zy[t] = acc[i][j];
        if (prob != nullptr && n < vp) prob[t * vp + n] = e[j];
      }
    }
  }
}

// dH[t, :] (or a split partial) = G[t, :] . W, in 64 x kDhBN tiles: dH has
// few rows per chunk, so narrow tiles give the vocabulary splits more
// workgroups for the same fp32 partials.
// blockIdx.z = vocabulary split: columns [z k_split, (z+1) k_split) of G and
// rows of W; with several splits `out` is split z's fp32 partial (part_stride apart).
template <typename T>
__global__ __launch_bounds__(256) void fma_dh_kernel(const float* __restrict__ G, int64_t vp, const T* __restrict__ W,
                                                     int64_t rows, int64_t d, int64_t v, int64_t k_split,
                                                     int64_t part_stride, int accumulate, T* __restrict__ out) {
  constexpr int JN = kDhBN / 16;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * kDhBN;
  const int64_t k_lo = static_cast<int64_t>(blockIdx.z) * k_split;
  const int64_t k_hi = k_lo + k_split < v ? k_lo + k_split : v;
  out += static_cast<int64_t>(blockIdx.z) * part_stride;
  float acc[4][JN];
  TileLoop<float, T, true, false, kDhBN>::run(G + k_lo, vp, W + k_lo * d, d, rows, d, k_hi > k_lo ? k_hi - k_lo : 0,
                                              m0, n0, acc);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = m0 + ty * 4 + i;
    if (t >= rows) continue;
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      const int64_t n = n0 + tx * JN + j;
      if (n < d) Elem<T>::st(out, t * d + n, accumulate ? Elem<T>::ld(out, t * d + n) + acc[i][j] : acc[i][j]);
    }
  }
}

// dW contribution of one chunk: partial[j, :] = sum_t G[t, j] H[t, :];
// DW_SINGLE writes it, DW_MID adds it to dW.
__global__ __launch_bounds__(256) void fma_dw_kernel(const float* __restrict__ G, int64_t vp, const float* __restrict__ H,
                                                     int64_t rows, int64_t d, int64_t v, float* __restrict__ out,
                                                     int mode) {
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * BN;
  float acc[4][4];
  TileLoop<float, float, false, false>::run(G, vp, H, d, v, d, rows, m0, n0, acc);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t j = m0 + ty * 4 + i;
    if (j >= v) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t n = n0 + tx * 4 + q;
      if (n >= d) continue;
      const int64_t o = j * d + n;
      out[o] = mode == DW_SINGLE ? acc[i][q] : out[o] + acc[i][q];
    }
  }
}

inline dim3 grid2(int64_t m, int64_t n) {
  return dim3(static_cast<unsigned>((m + BM - 1) / BM), static_cast<unsigned>((n + BN - 1) / BN));
}

}  // namespace

hipError_t fma_logits(const Plan& p, const Work& w, const ChunkArgs& a, int mode, hipStream_t s) {
  if (p.dtype != FLCE_F32) return hipErrorInvalidValue;
  float* prob = mode != LOGITS_STATS ? static_cast<float*>(w.prob) : nullptr;
  const float* lse_in = mode == LOGITS_GRAD_FROM_LSE ? a.lse_in : nullptr;
  // the grid spans the buffer's padded columns so that recompute mode clears them
  const int64_t cols = mode == LOGITS_GRAD_FROM_LSE ? p.vp : p.v;
  const dim3 grid(static_cast<unsigned>((a.rows + BM - 1) / BM), static_cast<unsigned>((cols + kLogitsBN - 1) / kLogitsBN));
  fma_logits_kernel<float><<<grid, 256, 0, s>>>(
      static_cast<const float*>(a.h), static_cast<const float*>(a.w), a.rows, p.d, p.v, p.vp, a.labels, w.zy, w.pm,
      w.ps, p.chunk, prob, lse_in, a.grad_out, w.nvalid, a.reduction, a.ignore_index);
  return hipGetLastError();
}

hipError_t fma_dh(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s) {
  if (p.dtype != FLCE_F32) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>((a.rows + BM - 1) / BM), static_cast<unsigned>((p.d + kDhBN - 1) / kDhBN),
            static_cast<unsigned>(p.dh_splits));
  const int64_t k_split = (p.v + p.dh_splits - 1) / p.dh_splits;
  float* out = p.dh_splits > 1 ? w.dhpart : static_cast<float*>(a.dh);
  fma_dh_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(w.prob), p.vp, static_cast<const float*>(a.w),
                                            a.rows, p.d, p.v, k_split, p.chunk * p.d,
                                            p.dh_splits == 1 && a.dh_accumulate, out);
  return hipGetLastError();
}

// dw_out (fp32) doubles as the accumulator: the first chunk writes, later chunks add.
hipError_t fma_dw(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s) {
  if (p.dtype != FLCE_F32) return hipErrorInvalidValue;
  float* out = static_cast<float*>(a.dw);
  const int mode = (a.dw_mode == DW_FIRST || a.dw_mode == DW_SINGLE) ? DW_SINGLE : DW_MID;
  fma_dw_kernel<<<grid2(p.v, p.d), 256, 0, s>>>(static_cast<const float*>(w.prob), p.vp,
                                               static_cast<const float*>(a.h), a.rows, p.d, p.v, out, mode);
  return hipGetLastError();
}

}  // namespace flce
