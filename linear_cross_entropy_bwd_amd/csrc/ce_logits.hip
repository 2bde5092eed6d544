// Cross-entropy on logits the caller already holds: per row the online
// log-sum-exp, the target logit and the loss, and optionally the gradient
// softmax - one-hot, written to a separate buffer or over the logits.  This
// is the step before the GEMM fusion (the LigerCrossEntropyLoss example of the
// lecture page "GPU MODE lecture 028 - Liger Kernel"): HBM-bound, one read of
// each row for the statistics and one read + write for the gradient.
#include "device_util.h"
#include "flce_internal.h"

#include <math.h>

namespace flce {

namespace {

constexpr int kCeThreads = 256;

// Running (max, sum of exp(z - max)) of a set of values; merging two is exact.
struct MaxSum {
  float m, s;
};

__device__ __forceinline__ MaxSum merge(MaxSum a, MaxSum b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return {m, 0.0f};
  return {m, a.s * fast_exp(a.m - m) + b.s * fast_exp(b.m - m)};
}

// 16 bytes of a row as floats: 8 bf16 or 4 fp32 values.
template <typename T>
struct Vec;
template <>
struct Vec<bf16_t> {
  static constexpr int kN = 8;
  static __device__ __forceinline__ void unpack(const uint4& u, float (&x)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float (&x)[8]) {
    uint4 u;
    u.x = pack_bf16x2(x[0], x[1]);
    u.y = pack_bf16x2(x[2], x[3]);
    u.z = pack_bf16x2(x[4], x[5]);
    u.w = pack_bf16x2(x[6], x[7]);
    return u;
  }
};
template <>
struct Vec<float> {
  static constexpr int kN = 4;
  static __device__ __forceinline__ void unpack(const uint4& u, float (&x)[4]) {
    x[0] = __uint_as_float(u.x);
    x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z);
    x[3] = __uint_as_float(u.w);
  }
  static __device__ __forceinline__ uint4 pack(const float (&x)[4]) {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
  }
};

template <typename T>
__device__ __forceinline__ void load_vec(const T* p, float (&x)[Vec<T>::kN]) {
  Vec<T>::unpack(*reinterpret_cast<const uint4*>(p), x);
}
template <typename T>
__device__ __forceinline__ void store_vec(T* p, const float (&x)[Vec<T>::kN]) {
  *reinterpret_cast<uint4*>(p) = Vec<T>::pack(x);
}

// (max, sum) of a whole workgroup; every thread gets the result.  red has one
// slot per wave.
template <int THREADS>
__device__ __forceinline__ MaxSum block_merge(MaxSum acc, MaxSum* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = 32; off > 0; off >>= 1) acc = merge(acc, {__shfl_xor(acc.m, off), __shfl_xor(acc.s, off)});
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  MaxSum t = red[0];
#pragma unroll
  for (int k = 1; k < THREADS / 64; ++k) t = merge(t, red[k]);
  return t;
}

// Streaming rows: one workgroup per row (grid-stride over rows), reading the
// row once for the statistics and once more for the gradient.  VEC: rows are
// read and written in 16-byte vectors (the row length in bytes is a multiple
// of 16), kUnroll of them in flight per thread; otherwise element by element.
// With lse_in the statistics pass is skipped (backward from the saved LSE).
template <typename T, bool VEC>
__global__ __launch_bounds__(kCeThreads) void ce_rows_kernel(
    const T* z, int64_t n, int64_t v, const int64_t* __restrict__ labels, int64_t ignore_index,
    int32_t reduction, const int32_t* __restrict__ nvalid, const float* __restrict__ lse_in,
    const float* __restrict__ grad_scale, float* __restrict__ lse_out, float* __restrict__ loss_rows, T* grad) {
  constexpr int kN = Vec<T>::kN;
  constexpr int kUnroll = 8;
  constexpr int64_t kStep = static_cast<int64_t>(kCeThreads) * kN;  // columns between a thread's vectors
  constexpr int64_t kSweep = kStep * kUnroll;
  __shared__ MaxSum red[kCeThreads / 64];
  __shared__ float row_lse;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t nv = *nvalid;
  const float rs = reduction == FLCE_SUM ? 1.0f : (nv > 0 ? 1.0f / static_cast<float>(nv) : 0.0f);
  const float go = grad_scale != nullptr ? *grad_scale : 1.0f;
  for (int64_t row = blockIdx.x; row < n; row += gridDim.x) {
    const T* zr = z + row * v;
    const int64_t y = labels[row];
    const bool valid = y != ignore_index;
    float lse;
    if (lse_in != nullptr) {
      lse = lse_in[row];
    } else {
      MaxSum acc = {-INFINITY, 0.0f};
      if constexpr (VEC) {
        // kUnroll vectors in flight per thread; those past the row end are
        // loaded from the last vector (unconditional loads: no wait between
        // them) and masked out of the running (max, sum)
        for (int64_t c = static_cast<int64_t>(tid) * kN; c < v; c += kSweep) {
          uint4 r[kUnroll];
#pragma unroll
          for (int u = 0; u < kUnroll; ++u)
            r[u] = *reinterpret_cast<const uint4*>(zr + min(c + u * kStep, v - kN));
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            float x[kN];
            Vec<T>::unpack(r[u], x);
            float lm = x[0];
#pragma unroll
            for (int k = 1; k < kN; ++k) lm = fmaxf(lm, x[k]);
            const float m = fmaxf(acc.m, lm);
            float ls = 0.0f;
#pragma unroll
            for (int k = 0; k < kN; ++k) ls += fast_exp(x[k] - m);
            const MaxSum next = {m, acc.s * fast_exp(acc.m - m) + ls};
            if (c + u * kStep < v) acc = next;
          }
        }
      } else {
        for (int64_t c = tid; c < v; c += kCeThreads) acc = merge(acc, {Elem<T>::ld(zr, c), 1.0f});
      }
      for (int off = 32; off > 0; off >>= 1)
        acc = merge(acc, {__shfl_xor(acc.m, off), __shfl_xor(acc.s, off)});
      if (lane == 0) red[wave] = acc;
      __syncthreads();
      if (tid == 0) {
        MaxSum t = red[0];
        for (int k = 1; k < kCeThreads / 64; ++k) t = merge(t, red[k]);
        const float l = t.m + logf(t.s);
        row_lse = l;
        lse_out[row] = l;
        const bool hit = valid && y >= 0 && y < v;
        loss_rows[row] = valid ? l - (hit ? Elem<T>::ld(zr, y) : 0.0f) : 0.0f;
      }
      __syncthreads();
      lse = row_lse;
    }
    if (grad != nullptr) {
      // g = (exp(z - lse) - [j = y]) * scale; the row may be the logits row itself
      const float sc = valid ? rs * go : 0.0f;
      T* gr = grad + row * v;
      if constexpr (VEC) {
        for (int64_t c = static_cast<int64_t>(tid) * kN; c < v; c += kSweep) {
          uint4 r[kUnroll];
#pragma unroll
          for (int u = 0; u < kUnroll; ++u)
            r[u] = *reinterpret_cast<const uint4*>(zr + min(c + u * kStep, v - kN));
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const int64_t cu = c + u * kStep;
            if (cu < v) {
              float x[kN];
              Vec<T>::unpack(r[u], x);
#pragma unroll
              for (int k = 0; k < kN; ++k) x[k] = (fast_exp(x[k] - lse) - (cu + k == y ? 1.0f : 0.0f)) * sc;
              store_vec(gr + cu, x);
            }
          }
        }
      } else {
        for (int64_t c = tid; c < v; c += kCeThreads)
          Elem<T>::st(gr, c, (fast_exp(Elem<T>::ld(zr, c) - lse) - (c == y ? 1.0f : 0.0f)) * sc);
      }
    }
    __syncthreads();  // row_lse and red are reused by the next row
  }
}

// Register-resident rows: the workgroup holds the whole row, NV 16-byte
// vectors per thread (vector i of thread t starts at column (i*THREADS + t)*kN,
// so a wave reads 1 KB contiguous per vector), kept packed as loaded.  One
// read of each row and, for the gradient, one write; every load of the row is
// in flight at once.  Rows must be 16-byte vectors end to end.
// The packed row is passed through an empty asm between the two sweeps, so the
// compiler re-unpacks it instead of keeping every unpacked float live (which
// would double the registers of bf16 rows).
template <int NV>
__device__ __forceinline__ void opaque(uint4 (&raw)[NV]) {
#pragma unroll
  for (int i = 0; i < NV; ++i) asm volatile("" : "+v"(raw[i].x), "+v"(raw[i].y), "+v"(raw[i].z), "+v"(raw[i].w));
}

template <typename T, int THREADS, int NV>
__global__ __launch_bounds__(THREADS) void ce_rows_resident_kernel(
    const T* z, int64_t n, int64_t v, const int64_t* __restrict__ labels, int64_t ignore_index, int32_t reduction,
    const int32_t* __restrict__ nvalid, const float* __restrict__ lse_in, const float* __restrict__ grad_scale,
    float* __restrict__ lse_out, float* __restrict__ loss_rows, T* grad) {
  constexpr int kN = Vec<T>::kN;
  constexpr int kStride = THREADS * kN;  // columns between a thread's consecutive vectors
  __shared__ MaxSum red[THREADS / 64];
  const int tid = threadIdx.x;
  const int32_t nv = *nvalid;
  const float rs = reduction == FLCE_SUM ? 1.0f : (nv > 0 ? 1.0f / static_cast<float>(nv) : 0.0f);
  const float go = grad_scale != nullptr ? *grad_scale : 1.0f;
  // v <= THREADS * NV * kN < 2^31 here, so column arithmetic fits 32 bits;
  // vector i of this thread covers columns c0 + i * kStride + [0, kN)
  const int c0 = tid * kN;
  const int lim = static_cast<int>(v) - c0;  // vector i exists iff i * kStride < lim
  for (int64_t row = blockIdx.x; row < n; row += gridDim.x) {
    const T* zr = z + row * v;
    const int64_t y = labels[row];
    const bool valid = y != ignore_index;
    const bool hit = valid && y >= 0 && y < v;
    // the one-hot column relative to this thread's first column; never matches when no column is hit
    const int yrel = hit ? static_cast<int>(y) - c0 : -1;
    // Every vector is loaded, those past the row end from the row's last
    // vector instead, and masked out below: a branch around each load would
    // make the compiler wait for one load before issuing the next.
    uint4 raw[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
      raw[i] = *reinterpret_cast<const uint4*>(zr + min(i * kStride + c0, static_cast<int>(v) - kN));
    // target logit: one address for every thread, read unconditionally (no
    // branch to wait at) and before any thread may overwrite the row in place
    const float zy = Elem<T>::ld(zr, hit ? y : 0);
    float lse;
    if (lse_in != nullptr) {
      lse = lse_in[row];
    } else {
      // one online sweep in load order, so each vector is consumed as it arrives
      MaxSum acc = {-INFINITY, 0.0f};
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        float x[kN];
        Vec<T>::unpack(raw[i], x);
        float lm = x[0];
#pragma unroll
        for (int k = 1; k < kN; ++k) lm = fmaxf(lm, x[k]);
        const float m = fmaxf(acc.m, lm);
        float ls = 0.0f;
#pragma unroll
        for (int k = 0; k < kN; ++k) ls += fast_exp(x[k] - m);
        const MaxSum next = {m, acc.s * fast_exp(acc.m - m) + ls};
        if (i * kStride < lim) acc = next;  // a select, not a branch
      }
      const MaxSum t = block_merge<THREADS>(acc, red);
      lse = t.m + logf(t.s);
      if (tid == 0) {
        lse_out[row] = lse;
        loss_rows[row] = valid ? lse - (hit ? zy : 0.0f) : 0.0f;
      }
      opaque(raw);  // the gradient sweep unpacks again rather than keeping this sweep's floats
    }
    if (grad != nullptr) {
      const float sc = valid ? rs * go : 0.0f;
      T* gr = grad + row * v;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (i * kStride < lim) {
          float x[kN];
          Vec<T>::unpack(raw[i], x);
#pragma unroll
          for (int k = 0; k < kN; ++k) x[k] = (fast_exp(x[k] - lse) - (yrel == i * kStride + k ? 1.0f : 0.0f)) * sc;
          store_vec(gr + i * kStride + c0, x);
        }
      }
    }
    __syncthreads();  // red is reused by the next row
  }
}

template <typename T, int THREADS, int NV>
void launch_resident(const CeArgs& a, unsigned grid, hipStream_t s) {
  ce_rows_resident_kernel<T, THREADS, NV><<<grid, THREADS, 0, s>>>(
      static_cast<const T*>(a.logits), a.n, a.v, a.labels, a.ignore_index, a.reduction, a.nvalid, a.lse_in,
      a.grad_scale, a.lse_out, a.loss_rows, static_cast<T*>(a.grad));
}

// Picks the resident kernel for rows of nvec 16-byte vectors: 256 threads for
// rows up to 4096 vectors (64 KB), 1024 threads up to 16384 vectors (256 KB,
// 64 VGPRs of row data per thread); returns false for longer rows.
template <typename T>
bool dispatch_resident(const CeArgs& a, int64_t nvec, unsigned grid, hipStream_t s) {
  if (nvec <= 256 * 1) launch_resident<T, 256, 1>(a, grid, s);
  else if (nvec <= 256 * 2) launch_resident<T, 256, 2>(a, grid, s);
  else if (nvec <= 256 * 4) launch_resident<T, 256, 4>(a, grid, s);
  else if (nvec <= 256 * 8) launch_resident<T, 256, 8>(a, grid, s);
  else if (nvec <= 256 * 16) launch_resident<T, 256, 16>(a, grid, s);
  else if (nvec <= 1024 * 8) launch_resident<T, 1024, 8>(a, grid, s);
  else if (nvec <= 1024 * 16) launch_resident<T, 1024, 16>(a, grid, s);
  else return false;
  return true;
}

template <typename T>
hipError_t launch_rows(const CeArgs& a, hipStream_t s) {
  const int64_t elem = static_cast<int64_t>(sizeof(T));
  const bool vec = (a.v * elem) % 16 == 0 && (reinterpret_cast<uintptr_t>(a.logits) % 16) == 0 &&
                   (a.grad == nullptr || (reinterpret_cast<uintptr_t>(a.grad) % 16) == 0);
  const unsigned grid = static_cast<unsigned>(a.n < 65536 ? a.n : 65536);
  const T* z = static_cast<const T*>(a.logits);
  T* g = static_cast<T*>(a.grad);
  // Rows that get a gradient run register-resident (a forward reads the row
  // once instead of twice; a backward from the saved LSE has every load of the
  // row in flight ahead of its stores).  A forward without a gradient streams:
  // several short workgroups per CU overlap one row's reduction with the next
  // row's loads.
  if (vec && a.grad != nullptr && dispatch_resident<T>(a, a.v * elem / 16, grid, s)) return hipGetLastError();
  if (vec)
    ce_rows_kernel<T, true><<<grid, kCeThreads, 0, s>>>(z, a.n, a.v, a.labels, a.ignore_index, a.reduction, a.nvalid,
                                                        a.lse_in, a.grad_scale, a.lse_out, a.loss_rows, g);
  else
    ce_rows_kernel<T, false><<<grid, kCeThreads, 0, s>>>(z, a.n, a.v, a.labels, a.ignore_index, a.reduction, a.nvalid,
                                                         a.lse_in, a.grad_scale, a.lse_out, a.loss_rows, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ce_rows(const CeArgs& a, hipStream_t s) {
  return a.dtype == FLCE_BF16 ? launch_rows<bf16_t>(a, s) : launch_rows<float>(a, s);
}

}  // namespace flce
